"""GPU parity: each C-ABI entry point against the CPU oracle on the same seeded inputs.

Layered contract:
  routing from given fp32 logits     -> ids bit-exact, gates within 1e-6, margin exact-ish
  projection logits                  -> within 1e-5 x max_e |l| per token
  routes from the projection         -> exact for every token whose fp64 margin exceeds the
                                        logit tolerance; near-tie tokens counted and checked valid
  alignment / capacity / stats       -> bit-exact
  expert FFN and combine, layer out  -> per-row max error <= rtol x rms(reference row),
                                        rtol 2e-2 (bf16, fp8 weights) / 1e-4 (fp32)
"""
import math
import sys

import numpy as np
import pytest
import torch

import top_routing_expert_router_amd as M
import workloads as W
from oracle import moe_oracle as O
from tests import harness as Hn

pytestmark = pytest.mark.gpu
DEV = "cuda"

# Sizes the oracle finishes in seconds while still spanning several tiles and a ragged tail.
SMALL = {
    "toy_fp32": W.TOY_FP32,
    "switch_capacity_bf16": W.SWITCH_BF16.with_(T=600),
    "mixtral_bf16": W.MIXTRAL_BF16.with_(T=300),
    "qwen3moe_bf16": W.QWEN3MOE_BF16.with_(T=700),
    "deepseekv3_fp8": W.DEEPSEEKV3_FP8.with_(T=200, N=24, H=1024, I=512),
}


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    M.lib()


_cache = {}


def inputs(w):
    key = w
    if key not in _cache:
        _cache.clear()
        big = w.H * w.I * w.N > 2e8
        d = W.layer_inputs(w, device="cpu", weights_device=DEV if big else "cpu")
        _cache[key] = (d, Hn.to_dev(d))
    return _cache[key]


# ------------------------------------------------------------------ routing

SPECIAL_ROWS = [
    [1.0, 1.0, 1.0, 0.5, 0.5, 0.5, 0.5, 0.5],
    [-0.0, 0.0, -1.0, -0.0, -2.0, 0.0, -0.0, 0.0],
    [float("nan"), 3.0, float("nan"), 1.0, 1.0, float("-inf"), 2.0, float("inf")],
    [float("nan")] * 7 + [7.0],
    [float("-inf")] * 8,
    [1e30, -1e30, 1e-30, -1e-30, 3.4e38, -3.4e38, 0.0, 1.0],
]


@pytest.mark.parametrize("name", ["toy_fp32", "mixtral_bf16", "qwen3moe_bf16", "deepseekv3_fp8"])
def test_route_from_logits_bit_exact(name):
    w = W.ALL[name]
    T = min(w.T, 4096)
    w = w.with_(T=T, near_tie_frac=0.05)
    lg = W.drawn_logits(w, T)
    if w.N >= 8:
        sp = torch.tensor(SPECIAL_ROWS, dtype=torch.float32)
        lg[:len(sp), :8] = sp
    _say("route_from_logits", name, T, w.N, w.k)
    cfg = Hn.config(w)
    b = Hn.route_buffers(w)
    b["logits"].copy_(lg)
    M.moe_route(cfg, None, None, None, b["logits"], b["ids"], b["gates"], b["margin"], flags=M.MOE_ROUTE_LOGITS_IN)
    torch.cuda.synchronize()
    ids, gates, margin = O.topk_route(lg.double().numpy(), w.k)
    got = b["ids"].cpu().numpy()
    assert np.array_equal(got, ids), np.argwhere(got != ids)[:5]
    gg = b["gates"].cpu().double().numpy()
    fin = np.isfinite(gates)
    assert np.array_equal(np.isfinite(gg), fin)
    assert np.max(np.abs(gg[fin] - gates[fin])) <= 1e-6
    gm = b["margin"].cpu().double().numpy()
    scale = np.nanmax(np.where(np.isfinite(lg.double().numpy()), np.abs(lg.double().numpy()), 0), axis=1)
    ok = np.isfinite(margin)
    assert np.array_equal(np.isfinite(gm), ok) or w.k == w.N
    assert np.all(np.abs(gm[ok] - margin[ok]) <= 1e-6 * np.maximum(scale[ok], 1.0))
    # the near-tie stress really is there
    assert np.count_nonzero(margin < 1e-3) >= int(0.04 * T)


@pytest.mark.parametrize("name", list(SMALL))
def test_route_projection(name):
    w = SMALL[name]
    d, dv = inputs(w)
    _say("route_projection", name, w)
    cfg = Hn.config(w)
    b = Hn.route_buffers(w)
    M.moe_route(cfg, dv["h"], dv["w_gate"], dv["bias"], b["logits"], b["ids"], b["gates"], b["margin"])
    torch.cuda.synchronize()
    l_ref = O.router_logits(Hn.f64(d["h"]), Hn.f64(d["w_gate"]), None if d["bias"] is None else Hn.f64(d["bias"]))
    l_gpu = b["logits"].cpu().double().numpy()
    scale = np.max(np.abs(l_ref), axis=1)
    err = np.max(np.abs(l_gpu - l_ref), axis=1) / scale
    assert err.max() <= 1e-5, err.max()
    ids_ref, gates_ref, margin_ref = O.topk_route(l_ref, w.k)
    near = margin_ref <= 2 * 1e-5 * scale
    got = b["ids"].cpu().numpy()
    diff = np.any(got != ids_ref, axis=1)
    _say(f"  near-tie tokens: {near.sum()}, of which routed differently: {(diff & near).sum()}")
    assert not np.any(diff & ~near), np.argwhere(diff & ~near)[:5]
    # every GPU route is a valid top-k of the GPU's own logits
    assert Hn.topk_valid(l_gpu, got).all()
    gg = b["gates"].cpu().double().numpy()
    same = ~diff
    assert np.max(np.abs(gg[same] - gates_ref[same])) <= 1e-6 + 2e-5 * scale.max()
    assert np.allclose(gg.sum(1), 1.0, atol=1e-6)


# ------------------------------------------------------------------ alignment and capacity

ALIGN_CASES = [
    ("toy", 64, 8, 2, 8, 0, 0, 0.0),
    ("switch_cap", 2048, 16, 1, 64, 5, 4, 1.1),
    ("mixtral", 4096, 8, 2, 64, 0, 0, 0.0),
    ("qwen3", 8192, 128, 8, 16, 0, 0, 0.3),
    ("deepseek", 16384, 256, 8, 64, 0, 0, 0.0),
    ("cap_zero", 5, 8, 1, 8, 5, 4, 0.0),
    ("skewed_cap", 3000, 32, 4, 32, 1, 1, 1.5),
    ("ragged", 1, 3, 2, 128, 0, 0, 0.0),
    ("max_t", 65536, 64, 8, 128, 3, 2, 0.5),
    # one-workgroup alignment up to 8192 routes, three kernels above: both sides of the
    # switch, 256 experts, invalid ids (one of them the last route)
    ("one_wg_max", 8192, 256, 1, 64, 3, 2, 0.8),
    ("three_kernel_min", 8193, 256, 1, 64, 3, 2, 0.8),
    ("one_wg_k8", 1000, 256, 8, 32, 0, 0, 0.3),
]


@pytest.mark.parametrize("case", ALIGN_CASES, ids=[c[0] for c in ALIGN_CASES])
def test_align_bit_exact(case):
    name, T, N, k, B, cn, cd, skew = case
    _say("align", case)
    w = W.Workload(name, T=T, H=128, N=N, k=k, I=128, B=B, act_dtype=W.BF16, expert_dtype=W.BF16,
                   cap_num=cn, cap_den=cd)
    ids = W.random_routes(T, N, k, seed=T + N, skew=skew)
    if name == "qwen3":  # a few invalid (replayed, out-of-range) ids
        ids[5, 0] = -1
        ids[77, 3] = N
        ids[100, 7] = 1 << 20
    if name in ("one_wg_max", "three_kernel_min", "one_wg_k8"):
        flat = ids.view(-1)
        flat[5] = -1
        flat[77] = N
        flat[-1] = 1 << 20
    cfg = Hn.config(w)
    b = Hn.run_align(cfg, w, ids.to(DEV))
    torch.cuda.synchronize()
    cap = O.capacity(T, k, N, cn, cd)
    kept = O.capacity_keep(ids.numpy(), N, cap)
    al = O.align(ids.numpy(), kept, N, B)
    assert np.array_equal(b["kept"].cpu().numpy().astype(bool), kept)
    assert np.array_equal(b["sorted"].cpu().numpy(), al["sorted_route_ids"])
    assert np.array_equal(b["blocks"].cpu().numpy(), al["block_expert"])
    assert np.array_equal(b["offsets"].cpu().numpy(), al["expert_offsets"])
    assert int(b["npad"].item()) == al["num_padded"]
    st = O.routing_stats(ids.numpy(), kept, N, cap)
    gs = b["stats"].cpu().numpy()
    assert np.array_equal(gs[:N], st["load"])
    X = M.STAT
    assert gs[N + X["kept"]] == st["kept_routes"]
    assert gs[N + X["dropped"]] == st["dropped_tokens"]
    assert gs[N + X["invalid"]] == st["invalid_routes"]
    assert gs[N + X["capacity"]] == st["capacity"]
    assert gs[N + X["max_load"]] == st["max_expert_load"]
    assert gs[N + X["min_load"]] == st["min_expert_load"]
    assert gs[N + X["num_padded"]] == al["num_padded"]
    assert gs[N + X["rerouted"]] == 0 and gs[N + X["unpicked"]] == 0 and gs[N + X["max_picks"]] == 0


# ------------------------------------------------------------------ expert FFN

def _oracle_alignment(w, seed=0):
    ids = W.random_routes(w.T, w.N, w.k, seed=seed, skew=0.3)
    cap = O.capacity(w.T, w.k, w.N, w.cap_num, w.cap_den)
    kept = O.capacity_keep(ids.numpy(), w.N, cap)
    al = O.align(ids.numpy(), kept, w.N, w.B)
    return ids, kept, al


# H an odd multiple of 128: the W2 tiles of the last weight n-tile are half past H, and the
# epilogue must store none of those columns (each chunk past H is staged, not stored); with
# I % 256 == 0 and one to four rounds of W2 tiles the micro-tile down-projection kernel runs too
ODD_H = {
    "odd_h_bf16": W.MIXTRAL_BF16.with_(T=300, H=640, I=384),
    "odd_h_bf16_micro": W.MIXTRAL_BF16.with_(T=12000, H=640, I=512),
    "odd_h_fp8": W.DEEPSEEKV3_FP8.with_(T=200, N=24, H=896, I=384),
}


@pytest.mark.parametrize("name", list(SMALL) + list(ODD_H))
def test_expert_ffn(name):
    """Every stored surface of the routed expert path, element by element: the W13 output
    (w13_out), the activation and the W2 output, each from the surface before it (bounds in
    tests/harness.py); rows of dropped routes untouched; w13_out changes no other bit."""
    w = SMALL[name] if name in SMALL else ODD_H[name]
    d, dv = inputs(w)
    _say("expert_ffn", name, w)
    ids, kept, al = _oracle_alignment(w)
    cfg = Hn.config(w)
    p_max, _ = M.moe_align_sizes(cfg)
    act_t = torch.float32 if w.act_dtype == W.F32 else torch.bfloat16
    sorted_d = torch.from_numpy(al["sorted_route_ids"].astype(np.int32)).to(DEV)
    offs_d = torch.from_numpy(al["expert_offsets"].astype(np.int32)).to(DEV)
    act = torch.zeros(p_max, w.I, dtype=act_t, device=DEV)
    y = torch.full((w.T * w.k, w.H), 7.0, dtype=act_t, device=DEV)
    M.moe_expert_ffn(cfg, dv["h"], sorted_d, offs_d, dv["w13"], dv["w2"], dv["w13_scale"], dv["w2_scale"], act, None, y)
    act2 = torch.zeros_like(act)
    y2 = torch.full_like(y, 7.0)
    w13o = torch.zeros(p_max, 2 * w.I, dtype=act_t, device=DEV)
    M.moe_expert_ffn(cfg, dv["h"], sorted_d, offs_d, dv["w13"], dv["w2"], dv["w13_scale"], dv["w2_scale"], act2, w13o,
                     y2)
    torch.cuda.synchronize()
    bits = torch.int32 if act_t == torch.float32 else torch.int16
    assert torch.equal(act.view(bits), act2.view(bits)) and torch.equal(y.view(bits), y2.view(bits))
    sorted_h = al["sorted_route_ids"]
    rows = np.nonzero(sorted_h < w.T * w.k)[0]          # padded rows that hold a kept route
    routes = sorted_h[rows]
    experts = ids.numpy().reshape(-1)[routes]
    x = Hn.f64(d["h"])[routes // w.k]
    Hn.check_expert_rows(w, x, experts, Hn.weights_f64(w, d, "w13"), Hn.weights_f64(w, d, "w2"),
                         Hn.f64(act)[rows], Hn.f64(y)[routes], got_w13=Hn.f64(w13o)[rows], say=_say)
    # rows of dropped routes are untouched
    dropped = np.nonzero(~kept)[0]
    if dropped.size:
        assert torch.all(y[torch.from_numpy(dropped).to(DEV)] == 7.0)


@pytest.mark.parametrize("name", ["toy_fp32", "mixtral_bf16", "deepseekv3_fp8"])
def test_shared_expert_identity_mode(name):
    # at least two 256-row tiles, so a tile that does not start at row 0 is checked
    w = SMALL[name].with_(n_shared=1, T=max(SMALL[name].T, 300))
    d = W.layer_inputs(w)
    dv = Hn.to_dev(d)
    _say("shared_expert", name)
    cfg = Hn.config(w)
    act_t = torch.float32 if w.act_dtype == W.F32 else torch.bfloat16
    act = torch.zeros(w.T, w.I, dtype=act_t, device=DEV)
    w13o = torch.zeros(w.T, 2 * w.I, dtype=act_t, device=DEV)
    y = torch.zeros(w.T, w.H, dtype=act_t, device=DEV)
    M.moe_expert_ffn(cfg, dv["h"], None, None, dv["shared_w13"], dv["shared_w2"], dv.get("shared_w13_scale"),
                     dv.get("shared_w2_scale"), act, w13o, y)
    torch.cuda.synchronize()
    s13, s2 = Hn.shared_f64(w, d, "w13"), Hn.shared_f64(w, d, "w2")
    Hn.check_expert_rows(w, Hn.f64(d["h"]), np.zeros(w.T, np.int64), lambda e: s13, lambda e: s2, Hn.f64(act),
                         Hn.f64(y), got_w13=Hn.f64(w13o), say=_say)


# ------------------------------------------------------------------ combine

@pytest.mark.parametrize("name", ["toy_fp32", "switch_capacity_bf16", "mixtral_bf16", "deepseekv3_fp8"])
def test_combine(name):
    w = W.ALL[name]
    T = min(w.T, 2048)
    w = w.with_(T=T)
    _say("combine", name)
    cfg = Hn.config(w)
    act_t = torch.float32 if w.act_dtype == W.F32 else torch.bfloat16
    y = W.random_rows(T * w.k, w.H, w.act_dtype, seed=1, name="y")
    res = W.random_rows(T, w.H, w.act_dtype, seed=2, name="res")
    res[3, :5] = -0.0
    sh = W.random_rows(T, w.H, w.act_dtype, seed=3, name="sh") if w.n_shared else None
    gates = W.random_gates(T, w.k, seed=4)
    g = torch.Generator().manual_seed(5)
    kept = (torch.rand(T * w.k, generator=g) > 0.3).to(torch.uint8)
    kept[3 * w.k:(3 + 1) * w.k] = 0  # token 3 fully dropped
    out = torch.empty(T, w.H, dtype=act_t, device=DEV)
    M.moe_combine(cfg, y.to(DEV), gates.to(DEV), kept.to(DEV), None if sh is None else sh.to(DEV), res.to(DEV), out)
    torch.cuda.synchronize()
    yd = {r: Hn.f64(y[r]) for r in range(T * w.k)}
    ref = O.combine(yd, gates.double().numpy(), kept.numpy().astype(bool), T, w.H,
                    shared=None if sh is None else Hn.f64(sh), residual=Hn.f64(res))
    got = Hn.f64(out)
    # fp32 accumulation of at most k+2 terms, then one round-to-nearest to the act dtype:
    # |error| <= half an ulp of the result (2^-8 relative in bf16, 2^-24 in fp32) + accumulation slack
    mag = np.abs(Hn.f64(res)) + (0 if sh is None else np.abs(Hn.f64(sh)))
    for j in range(w.k):
        mag = mag + np.abs(gates[:, j:j + 1].double().numpy() * Hn.f64(y[j::w.k]))
    half_ulp = 2.0 ** (-24 if w.act_dtype == W.F32 else -8)
    bound = half_ulp * np.abs(ref) + (w.k + 2) * 2.0 ** -24 * mag * (1 + half_ulp)
    excess = np.abs(got - ref) - bound
    assert excess.max() <= 0, (excess.max(), np.unravel_index(excess.argmax(), excess.shape))
    if sh is None:
        # fully dropped token: its residual row, bit for bit (including -0)
        assert torch.equal(out[3].cpu().view(torch.int16 if act_t == torch.bfloat16 else torch.int32),
                           res[3].view(torch.int16 if act_t == torch.bfloat16 else torch.int32))


# ------------------------------------------------------------------ whole layer

def run_forward(w, dv, trace=True):
    cfg = Hn.config(w)
    p_max, n_blocks = M.moe_align_sizes(cfg)
    act_t = torch.float32 if w.act_dtype == W.F32 else torch.bfloat16
    ws = torch.empty(M.moe_workspace_size(cfg, M.MOE_OP_FORWARD), dtype=torch.uint8, device=DEV)
    out = torch.empty(w.T, w.H, dtype=act_t, device=DEV)
    tr = None
    if trace:
        tr = dict(logits=torch.empty(w.T, w.N, device=DEV), topk_ids=torch.empty(w.T, w.k, dtype=torch.int32, device=DEV),
                  topk_gates=torch.empty(w.T, w.k, device=DEV), margin=torch.empty(w.T, device=DEV),
                  route_kept=torch.empty(w.T * w.k, dtype=torch.uint8, device=DEV),
                  sorted_route_ids=torch.empty(p_max, dtype=torch.int32, device=DEV),
                  block_expert=torch.empty(n_blocks, dtype=torch.int32, device=DEV),
                  expert_offsets=torch.empty(w.N + 1, dtype=torch.int32, device=DEV),
                  num_padded=torch.empty(1, dtype=torch.int32, device=DEV),
                  stats=torch.empty(w.N + M.STATS_EXTRA, dtype=torch.int32, device=DEV),
                  y_route=torch.empty(w.T * w.k, w.H, dtype=act_t, device=DEV))
    wts = {k: dv.get(k) for k in ("w_gate", "w13", "w2", "w13_scale", "w2_scale", "shared_w13", "shared_w2",
                                  "shared_w13_scale", "shared_w2_scale")}
    wts["logit_bias"] = dv.get("bias")
    M.moe_forward(cfg, wts, dv["h"], dv["residual"], out, tr, ws)
    torch.cuda.synchronize()
    return out, tr


# degenerate shapes of the layer: one expert (a plain SwiGLU FFN per token), every token on
# every expert (k = N, margin +inf), one token over 64 experts (56 of them empty), and fp8
# weights with two experts and a shared expert
DEGENERATE = {
    "single_expert": W.MIXTRAL_BF16.with_(T=70, H=256, N=1, k=1, I=256, B=16),
    "k_equals_n": W.MIXTRAL_BF16.with_(T=100, H=256, N=4, k=4, I=256, B=8),
    "one_token_64_experts": W.QWEN3MOE_BF16.with_(T=1, H=512, N=64, k=8, I=384, B=16),
    "fp8_two_experts_shared": W.DEEPSEEKV3_FP8.with_(T=33, H=256, N=2, k=2, I=256, B=64),
}


@pytest.mark.parametrize("name", list(SMALL) + list(DEGENERATE))
def test_forward_end_to_end(name):
    w = SMALL[name] if name in SMALL else DEGENERATE[name]
    d, dv = inputs(w)
    _say("forward", name, w)
    out, tr = run_forward(w, dv)
    res = O.moe_forward(Hn.f64(d["h"]), Hn.f64(d["w_gate"]), Hn.weights_f64(w, d, "w13"), Hn.weights_f64(w, d, "w2"),
                        k=w.k, B=w.B, cap_num=w.cap_num, cap_den=w.cap_den,
                        bias=None if d["bias"] is None else Hn.f64(d["bias"]), residual=Hn.f64(d["residual"]),
                        shared_w13=Hn.shared_f64(w, d, "w13") if w.n_shared else None,
                        shared_w2=Hn.shared_f64(w, d, "w2") if w.n_shared else None)
    scale = np.max(np.abs(res["logits"]), axis=1)
    near = res["margin"] <= 2e-5 * scale
    ids = tr["topk_ids"].cpu().numpy()
    diff = np.any(ids != res["ids"], axis=1)
    _say(f"  near-tie {near.sum()}, differing {diff.sum()}")
    assert not np.any(diff & ~near)
    # capacity and alignment: the oracle's steps on the GPU's own ids, bit-exact, no exclusion
    cap = O.capacity(w.T, w.k, w.N, w.cap_num, w.cap_den)
    kept_ref = O.capacity_keep(ids.astype(np.int64), w.N, cap)
    al = O.align(ids.astype(np.int64), kept_ref, w.N, w.B)
    assert np.array_equal(tr["route_kept"].cpu().numpy().astype(bool), kept_ref)
    assert np.array_equal(tr["sorted_route_ids"].cpu().numpy(), al["sorted_route_ids"])
    assert np.array_equal(tr["expert_offsets"].cpu().numpy(), al["expert_offsets"])
    assert np.array_equal(tr["block_expert"].cpu().numpy(), al["block_expert"])
    assert int(tr["num_padded"].item()) == al["num_padded"]
    if not diff.any():
        assert np.array_equal(kept_ref, res["kept"])
    good = ~diff
    err = Hn.row_rel_err(Hn.f64(out)[good], res["out"][good])
    _say(f"  max out row err {err.max():.3e}")
    assert err.max() <= Hn.tol(w)
    # a fully dropped token outputs its residual bit for bit
    kept = tr["route_kept"].cpu().numpy().reshape(w.T, w.k).astype(bool)
    gone = np.nonzero(~kept.any(1))[0]
    if gone.size and not w.n_shared:
        idx = torch.from_numpy(gone).to(DEV)
        assert torch.equal(out[idx], dv["residual"][idx])


@pytest.mark.parametrize("name", ["mixtral_bf16", "qwen3moe_bf16", "deepseekv3_fp8"])
def test_route_without_logits_out(name):
    """MOE_ROUTE_NO_LOGITS_OUT: the same ids, gates and margins as with the logits written,
    and the logits buffer untouched."""
    w = SMALL[name]
    _say("route without logits out", name)
    h = W.hidden_states(w, device=DEV)
    wg = W.router_weight(w, device=DEV)
    cfg = Hn.config(w)
    a, b = Hn.route_buffers(w), Hn.route_buffers(w)
    M.moe_route(cfg, h, wg, None, a["logits"], a["ids"], a["gates"], a["margin"])
    b["logits"].fill_(7.0)
    M.moe_route(cfg, h, wg, None, b["logits"], b["ids"], b["gates"], b["margin"], flags=M.MOE_ROUTE_NO_LOGITS_OUT)
    c = Hn.route_buffers(w)
    M.moe_route(cfg, h, wg, None, None, c["ids"], c["gates"], c["margin"], flags=M.MOE_ROUTE_NO_LOGITS_OUT)
    torch.cuda.synchronize()
    assert torch.all(b["logits"] == 7.0)
    for x in (b, c):
        assert torch.equal(x["ids"], a["ids"])
        assert torch.equal(x["gates"].view(torch.int32), a["gates"].view(torch.int32))
        assert torch.equal(x["margin"].view(torch.int32), a["margin"].view(torch.int32))


@pytest.mark.parametrize("T,N,H", [(300, 256, 1024), (777, 200, 2048), (16384, 256, 7168)])
def test_route_projection_many_experts(T, N, H):
    """More than 128 experts take the kernel that stages W_g once per 32 or 64 tokens:
    logits within 1e-5 x max|l| of the oracle, routes exact away from near ties, and the
    bits of a token's logits the same whether it runs in a 64-token or a 32-token tile."""
    w = W.DEEPSEEKV3_FP8.with_(T=T, N=N, H=H)
    _say("route_projection many experts", T, N, H)
    h = W.hidden_states(w, device=DEV)
    wg = W.router_weight(w, device=DEV)
    cfg = Hn.config(w)
    b = Hn.route_buffers(w)
    M.moe_route(cfg, h, wg, None, b["logits"], b["ids"], b["gates"], b["margin"])
    torch.cuda.synchronize()
    rows = np.arange(T) if T <= 1024 else np.sort(np.random.default_rng(3).choice(T, 512, replace=False))
    l_ref = O.router_logits(Hn.f64(h[torch.from_numpy(rows).to(DEV)]), Hn.f64(wg))
    l_gpu = b["logits"].cpu().double().numpy()[rows]
    scale = np.max(np.abs(l_ref), axis=1)
    err = np.max(np.abs(l_gpu - l_ref), axis=1) / scale
    assert err.max() <= 1e-5, err.max()
    ids_ref, _, margin_ref = O.topk_route(l_ref, w.k)
    ids = b["ids"].cpu().numpy()[rows]
    diff = np.any(ids != ids_ref, axis=1)
    assert not np.any(diff & ~(margin_ref <= 2e-5 * scale))
    assert Hn.topk_valid(b["logits"].cpu().double().numpy()[rows], ids).all()
    # the same tokens alone (a smaller grid, 32-token tiles): the same logit bits
    sub = torch.from_numpy(rows[:100]).to(DEV)
    w2 = w.with_(T=100)
    b2 = Hn.route_buffers(w2)
    M.moe_route(Hn.config(w2), h[sub].contiguous(), wg, None, b2["logits"], b2["ids"], b2["gates"], b2["margin"])
    torch.cuda.synchronize()
    assert torch.equal(b2["logits"].view(torch.int32), b["logits"][sub].view(torch.int32))
    assert torch.equal(b2["ids"], b["ids"][sub])
