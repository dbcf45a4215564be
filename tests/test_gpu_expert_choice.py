"""Expert-choice routing on the GPU against the oracle.

"Mixture-of-experts routing & LLM repeatability", paragraph on expert-choice routing:
each expert takes its highest-scoring tokens from the whole batch.  "Mixture-of-Experts
Routing at Inference Time", "Integration: where routing lives in a serving stack",
paragraph on expert-choice routing: up to each expert's capacity; a token may be picked
by no expert.

Layered like the token-choice contract:
  logits from the projection       -> within 1e-5 x max_e |l| per token
  scores from the GPU's logits     -> within 2e-6 relative of the oracle's softmax, and
                                      bitwise the token-choice gates with renormalize = 0
  picks from the GPU's scores      -> tokens, slots and alignment bit-exact, margin within
                                      one fp32 ulp of the oracle's
  picks from the fp64 logits       -> equal except for tokens within rounding of the cut
  layer output (oracle replays the GPU's scores) -> per-row error <= rtol x rms(row); a
                                      token no expert picked outputs its residual bitwise
"""
import numpy as np
import pytest
import torch

import top_routing_expert_router_amd as M
import workloads as W
from oracle import moe_oracle as O
from tests import harness as Hn
from tests.test_gpu_parity import inputs, _say

pytestmark = pytest.mark.gpu
DEV = "cuda"

# Sizes the oracle finishes in seconds; the Mixtral shape spans two m-tiles per expert
# (275 picks in a 320-row segment) and two key slots per thread in the selection.
SMALL = {
    "toy_ec_fp32": W.TOY_EC_FP32,
    "mixtral_ec_bf16": W.MIXTRAL_EC_BF16.with_(T=1100),
    "qwen3moe_ec_bf16": W.QWEN3MOE_EC_BF16.with_(T=700),
    "deepseekv3_ec_fp8": W.DEEPSEEKV3_EC_FP8.with_(T=200, N=24, H=1024, I=512),
    # capacity factor 1/2: fewer picks than tokens, so many tokens go unpicked
    "mixtral_ec_half_bf16": W.MIXTRAL_EC_BF16.with_(name="mixtral_ec_half_bf16", T=600, cap_num=1, cap_den=2),
}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    M.lib()


def _bits(t):
    return t.contiguous().view(torch.int32) if t.dtype == torch.float32 else t.contiguous().view(torch.int16)


def _route_buffers(w, C):
    return dict(logits=torch.empty(w.T, w.N, device=DEV), scores=torch.empty(w.T, w.N, device=DEV),
                tokens=torch.full((max(w.N * C, 1),), -7, dtype=torch.int32, device=DEV),
                slot=torch.full((w.T, w.N), -7, dtype=torch.int32, device=DEV),
                margin=torch.full((w.N,), -7.0, device=DEV))


def _route(w, dv=None, logits=None):
    cfg = Hn.config(w)
    C, seg = M.moe_expert_choice_sizes(cfg)
    b = _route_buffers(w, C)
    if logits is not None:
        b["logits"].copy_(logits)
        M.moe_route_expert_choice(cfg, None, None, None, b["logits"], b["scores"], b["tokens"], b["slot"],
                                  b["margin"], flags=M.MOE_ROUTE_LOGITS_IN)
    else:
        M.moe_route_expert_choice(cfg, dv["h"], dv["w_gate"], dv["bias"], b["logits"], b["scores"], b["tokens"],
                                  b["slot"], b["margin"])
    torch.cuda.synchronize()
    return cfg, C, seg, b


def _check_scores(b):
    """GPU scores vs the oracle's softmax of the GPU's own logits."""
    l = b["logits"].cpu().double().numpy()
    ref = O.expert_scores(l)
    got = b["scores"].cpu().double().numpy()
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.all(np.abs(got[ok] - ref[ok]) <= 2e-6 * ref[ok]), np.max(np.abs(got[ok] - ref[ok]) / np.maximum(ref[ok], 1e-300))
    return got


def _check_picks(b, C, N):
    """Picks of the GPU's scores, bit for bit, and the margin within an fp32 ulp."""
    S = b["scores"].cpu().double().numpy()
    tok, slot, margin = O.expert_choice_select(S, C)
    got_tok = b["tokens"][:N * C].cpu().numpy().reshape(N, C)
    assert np.array_equal(got_tok, tok), np.argwhere(got_tok != tok)[:5]
    got_slot = b["slot"].cpu().numpy()
    assert np.array_equal(got_slot, slot), np.argwhere(got_slot != slot)[:5]
    gm = b["margin"].cpu().numpy()
    want = margin.astype(np.float32)
    assert np.array_equal(np.isnan(gm), np.isnan(want))
    inf = np.isinf(want)
    assert np.array_equal(gm[inf], want[inf])
    fin = np.isfinite(want)
    assert np.all(np.abs(gm[fin] - want[fin]) <= np.spacing(np.abs(want[fin]))), (gm[fin], want[fin])
    return tok, slot


# ------------------------------------------------------------------ routing


@pytest.mark.parametrize("name", list(SMALL))
def test_scores_and_picks_from_the_projection(name):
    w = SMALL[name]
    d, dv = inputs(w)
    _say("expert choice route", name, w.T, w.N, w.k)
    cfg, C, seg, b = _route(w, dv)
    l_ref = O.router_logits(Hn.f64(d["h"]), Hn.f64(d["w_gate"]), None if d["bias"] is None else Hn.f64(d["bias"]))
    l_gpu = b["logits"].cpu().double().numpy()
    scale = np.max(np.abs(l_ref), axis=1)
    assert (np.max(np.abs(l_gpu - l_ref), axis=1) / scale).max() <= 1e-5
    S = _check_scores(b)
    tok, _ = _check_picks(b, C, w.N)
    # a token's top-k scores are bitwise its token-choice gates without renormalisation
    wt = w.with_(routing="token_choice", renormalize=0)
    rb = Hn.route_buffers(wt)
    rb["logits"].copy_(b["logits"])
    M.moe_route(Hn.config(wt), None, None, None, rb["logits"], rb["ids"], rb["gates"], rb["margin"],
                flags=M.MOE_ROUTE_LOGITS_IN)
    torch.cuda.synchronize()
    assert torch.equal(_bits(torch.gather(b["scores"], 1, rb["ids"].long())), _bits(rb["gates"]))
    # end to end: the picks from the exact fp64 logits differ only within rounding of the cut
    S_ref = O.expert_scores(l_ref)
    tok_ref, _, _ = O.expert_choice_select(S_ref, C)
    near = 0
    for e in range(w.N):
        a, r = set(tok[e].tolist()), set(tok_ref[e].tolist())
        if a == r or C == 0:
            continue
        cut = np.sort(S_ref[:, e])[::-1][C - 1]
        for t in a ^ r:
            assert abs(S_ref[t, e] - cut) <= 1e-4 * cut, (e, t, S_ref[t, e], cut)
            near += 1
    _say(f"  C={C}, picks differing within rounding of the cut: {near}")


def _drawn(T, N, kind, seed):
    g = torch.Generator().manual_seed(seed)
    lg = torch.randn(T, N, generator=g) * 0.905
    if kind == "ties":  # a few distinct rows, each token a copy: exact score ties everywhere
        base = torch.randn(7, N, generator=g) * 0.905
        base[3] = base[1]
        lg = base[torch.randint(0, 7, (T,), generator=g)]
    elif kind == "nan":
        lg[torch.rand(T, N, generator=g) < 0.01] = float("nan")
        lg[5] = float("nan")
        lg[9, 0] = float("inf")
        lg[11] = -0.0
    return lg.contiguous()


CASES = [
    # (T, N, k, cap_num, cap_den, kind)
    (1, 8, 2, 0, 0, "drawn"),        # C = 0: nothing picked
    (5, 8, 8, 0, 0, "drawn"),        # C = T: every token picked by every expert
    (700, 1, 1, 0, 0, "ties"),       # one expert taking every token
    (1000, 16, 2, 5, 4, "ties"),     # one key slot per thread, heavy ties at every cut
    (3000, 8, 2, 0, 0, "ties"),      # ragged T across key slots
    (4096, 256, 8, 0, 0, "drawn"),   # 256 experts
    (20000, 64, 4, 3, 2, "nan"),     # NaN, inf and -0 logits
    (65536, 8, 2, 0, 0, "drawn"),    # the largest T: 64 key slots per thread
]


@pytest.mark.parametrize("case", CASES, ids=[f"T{c[0]}_N{c[1]}_k{c[2]}_{c[5]}" for c in CASES])
def test_picks_from_given_logits(case):
    T, N, k, cn, cd, kind = case
    w = W.MIXTRAL_EC_BF16.with_(T=T, N=N, k=k, cap_num=cn, cap_den=cd)
    _say("expert choice picks", case)
    cfg, C, seg, b = _route(w, logits=_drawn(T, N, kind, seed=T + N))
    _check_scores(b)
    tok, slot = _check_picks(b, C, N)
    if C == 0:
        assert np.all(slot == -1)
    if C == T:
        assert np.all(slot >= 0)


# ------------------------------------------------------------------ alignment


def _align(cfg, w, b, C, seg):
    P, nb = M.moe_align_sizes(cfg)
    a = dict(sorted=torch.full((max(P, 1),), -7, dtype=torch.int32, device=DEV),
             blocks=torch.full((max(nb, 1),), -7, dtype=torch.int32, device=DEV),
             offsets=torch.full((w.N + 1,), -7, dtype=torch.int32, device=DEV),
             npad=torch.full((1,), -7, dtype=torch.int32, device=DEV),
             stats=torch.full((w.N + M.STATS_EXTRA,), -7, dtype=torch.int32, device=DEV))
    M.moe_align_expert_choice(cfg, b["tokens"], b["slot"], a["sorted"], a["blocks"], a["offsets"], a["npad"],
                              a["stats"])
    torch.cuda.synchronize()
    return P, nb, a


@pytest.mark.parametrize("case", CASES[:5], ids=[f"T{c[0]}_N{c[1]}_k{c[2]}" for c in CASES[:5]])
def test_align_bit_exact(case):
    T, N, k, cn, cd, kind = case
    w = W.MIXTRAL_EC_BF16.with_(T=T, N=N, k=k, cap_num=cn, cap_den=cd)
    cfg, C, seg, b = _route(w, logits=_drawn(T, N, kind, seed=3 * T + N))
    P, nb, a = _align(cfg, w, b, C, seg)
    tok, slot, _ = O.expert_choice_select(b["scores"].cpu().double().numpy(), C)
    al = O.expert_choice_align(tok, T, w.B)
    assert P == al["num_padded"] and nb == al["block_expert"].size
    assert np.array_equal(a["sorted"][:P].cpu().numpy(), al["sorted_tokens"])
    assert np.array_equal(a["blocks"][:nb].cpu().numpy(), al["block_expert"])
    assert np.array_equal(a["offsets"].cpu().numpy(), al["expert_offsets"])
    assert int(a["npad"].item()) == P
    st = a["stats"].cpu().numpy()
    picks = np.count_nonzero(slot >= 0, axis=1)
    x = st[N:]
    assert np.all(st[:N] == C)
    assert x[M.STAT["kept"]] == N * C and x[M.STAT["capacity"]] == C and x[M.STAT["num_padded"]] == P
    assert x[M.STAT["max_load"]] == C and x[M.STAT["min_load"]] == C
    assert x[M.STAT["dropped"]] == 0 and x[M.STAT["invalid"]] == 0 and x[M.STAT["rerouted"]] == 0
    assert x[M.STAT["unpicked"]] == np.count_nonzero(picks == 0)
    assert x[M.STAT["max_picks"]] == picks.max()


# ------------------------------------------------------------------ layer


def _trace(cfg, w, C, act_t):
    P, nb = M.moe_align_sizes(cfg)
    return dict(logits=torch.empty(w.T, w.N, device=DEV), scores=torch.empty(w.T, w.N, device=DEV),
                choice_tokens=torch.empty(max(w.N * C, 1), dtype=torch.int32, device=DEV),
                choice_slot=torch.empty(w.T, w.N, dtype=torch.int32, device=DEV),
                choice_margin=torch.empty(w.N, device=DEV),
                sorted_route_ids=torch.empty(max(P, 1), dtype=torch.int32, device=DEV),
                block_expert=torch.empty(max(nb, 1), dtype=torch.int32, device=DEV),
                expert_offsets=torch.empty(w.N + 1, dtype=torch.int32, device=DEV),
                num_padded=torch.empty(1, dtype=torch.int32, device=DEV),
                stats=torch.empty(w.N + M.STATS_EXTRA, dtype=torch.int32, device=DEV),
                act=torch.empty(max(P, 1), w.I, dtype=act_t, device=DEV),
                y_route=torch.empty(max(P, 1), w.H, dtype=act_t, device=DEV))


def _weights(dv):
    wts = {k: dv.get(k) for k in Hn.WEIGHT_KEYS}
    wts["logit_bias"] = dv.get("bias")
    return wts


def _forward(w, dv):
    cfg = Hn.config(w)
    C, _ = M.moe_expert_choice_sizes(cfg)
    act_t = torch.float32 if w.act_dtype == W.F32 else torch.bfloat16
    ws = torch.empty(M.moe_workspace_size(cfg, M.MOE_OP_FORWARD), dtype=torch.uint8, device=DEV)
    out = torch.empty(w.T, w.H, dtype=act_t, device=DEV)
    tr = _trace(cfg, w, C, act_t)
    M.moe_forward(cfg, _weights(dv), dv["h"], dv["h"], out, tr, ws)
    torch.cuda.synchronize()
    return cfg, C, out, tr


@pytest.mark.parametrize("name", list(SMALL))
def test_forward_end_to_end(name):
    w = SMALL[name]
    d, dv = inputs(w)
    _say("expert choice forward", name)
    cfg, C, out, tr = _forward(w, dv)
    S = tr["scores"].cpu().double().numpy()
    res = O.expert_choice_forward(Hn.f64(d["h"]), Hn.f64(d["w_gate"]), Hn.weights_f64(w, d, "w13"),
                                  Hn.weights_f64(w, d, "w2"), k=w.k, B=w.B, cap_num=w.cap_num, cap_den=w.cap_den,
                                  residual=Hn.f64(d["residual"]),
                                  shared_w13=Hn.shared_f64(w, d, "w13") if w.n_shared else None,
                                  shared_w2=Hn.shared_f64(w, d, "w2") if w.n_shared else None, scores=S)
    assert res["cap"] == C
    assert np.array_equal(tr["choice_tokens"][:w.N * C].cpu().numpy().reshape(w.N, C), res["tokens"])
    assert np.array_equal(tr["choice_slot"].cpu().numpy(), res["slot"])
    P = res["align"]["num_padded"]
    assert np.array_equal(tr["sorted_route_ids"][:P].cpu().numpy(), res["align"]["sorted_tokens"])
    assert np.array_equal(tr["expert_offsets"].cpu().numpy(), res["align"]["expert_offsets"])
    st = tr["stats"].cpu().numpy()[w.N:]
    assert st[M.STAT["unpicked"]] == res["stats"]["unpicked_tokens"]
    assert st[M.STAT["max_picks"]] == res["stats"]["max_picks"]
    err = Hn.row_rel_err(Hn.f64(out), res["out"])
    _say(f"  C={C}, unpicked {res['stats']['unpicked_tokens']}, max row err {err.max():.3e}")
    assert err.max() <= Hn.tol(w)
    unpicked = np.count_nonzero(res["slot"] >= 0, axis=1) == 0
    if not w.n_shared and unpicked.any():
        idx = torch.from_numpy(np.nonzero(unpicked)[0]).to(DEV)
        assert torch.equal(_bits(out[idx]), _bits(dv["h"][idx]))  # the dual failure: h alone


@pytest.mark.parametrize("name", list(SMALL))
def test_forward_trace_matches_standalone_calls_and_repeats(name):
    w = SMALL[name]
    d, dv = inputs(w)
    _say("expert choice trace", name)
    cfg, C, out, tr = _forward(w, dv)
    _, _, out2, _ = _forward(w, dv)
    assert torch.equal(_bits(out2), _bits(out))  # same inputs, same bits
    _, _, seg, b = _route(w, dv)
    for a, k in (("logits", "logits"), ("scores", "scores"), ("choice_slot", "slot"), ("choice_margin", "margin")):
        assert torch.equal(_bits(tr[a]) if tr[a].is_floating_point() else tr[a],
                           _bits(b[k]) if b[k].is_floating_point() else b[k]), a
    assert torch.equal(tr["choice_tokens"][:w.N * C], b["tokens"][:w.N * C])
    P, nb, a = _align(cfg, w, b, C, seg)
    for x, y in (("sorted_route_ids", "sorted"), ("block_expert", "blocks"), ("expert_offsets", "offsets"),
                 ("num_padded", "npad"), ("stats", "stats")):
        assert torch.equal(tr[x][:a[y].numel()], a[y][:tr[x].numel()]), x
    act = torch.zeros_like(tr["act"])
    y = torch.zeros_like(tr["y_route"])
    M.moe_expert_ffn(cfg, dv["h"], a["sorted"], a["offsets"], dv["w13"], dv["w2"], dv.get("w13_scale"),
                     dv.get("w2_scale"), act, None, y)
    torch.cuda.synchronize()
    real = (a["sorted"][:P] < w.T)
    assert torch.equal(_bits(act[:P][real]), _bits(tr["act"][:P][real]))
    assert torch.equal(_bits(y[:P][real]), _bits(tr["y_route"][:P][real]))
    shared = None
    act_t = out.dtype
    if w.n_shared:
        sact = torch.empty(w.T, w.I, dtype=act_t, device=DEV)
        shared = torch.empty(w.T, w.H, dtype=act_t, device=DEV)
        M.moe_expert_ffn(cfg, dv["h"], None, None, dv["shared_w13"], dv["shared_w2"], dv.get("shared_w13_scale"),
                         dv.get("shared_w2_scale"), sact, None, shared)
    out3 = torch.empty_like(out)
    M.moe_combine_expert_choice(cfg, y, b["scores"], b["slot"], shared, dv["h"], out3)
    torch.cuda.synchronize()
    assert torch.equal(_bits(out3), _bits(out))


def test_forward_with_no_capacity_outputs_the_residual():
    # 3 tokens, 8 experts, k = 1: C = floor(3 / 8) = 0 -- no expert picks anything
    w = W.MIXTRAL_EC_BF16.with_(T=3, k=1, H=256, I=256)
    d, dv = inputs(w)
    cfg, C, out, tr = _forward(w, dv)
    assert C == 0
    assert torch.equal(_bits(out), _bits(dv["h"]))
    st = tr["stats"].cpu().numpy()[w.N:]
    assert st[M.STAT["unpicked"]] == 3 and st[M.STAT["kept"]] == 0 and int(tr["num_padded"].item()) == 0


def test_full_size_mixtral_expert_choice():
    w = W.MIXTRAL_EC_BF16
    d, dv = inputs(w)
    _say("expert choice full size", w.T, w.N, w.k)
    cfg, C, out, tr = _forward(w, dv)
    S = tr["scores"].cpu().double().numpy()
    tok, slot, _ = O.expert_choice_select(S, C)
    assert np.array_equal(tr["choice_tokens"][:w.N * C].cpu().numpy().reshape(w.N, C), tok)
    assert np.array_equal(tr["choice_slot"].cpu().numpy(), slot)
    picks = np.count_nonzero(slot >= 0, axis=1)
    g = np.random.default_rng(0)
    sample = np.unique(np.concatenate([g.choice(w.T, 24, replace=False), np.nonzero(picks == 0)[0][:4],
                                       np.nonzero(picks == picks.max())[0][:4]]))
    res = O.expert_choice_forward(Hn.f64(d["h"]), Hn.f64(d["w_gate"]), Hn.weights_f64(w, d, "w13"),
                                  Hn.weights_f64(w, d, "w2"), k=w.k, B=w.B, residual=Hn.f64(d["residual"]),
                                  scores=S, tokens=sample)
    err = Hn.row_rel_err(Hn.f64(out[torch.from_numpy(sample).to(DEV)]), res["out"])
    _say(f"  C={C}, unpicked {int(np.count_nonzero(picks == 0))}, max picks {picks.max()}, "
         f"sampled max row err {err.max():.3e}")
    assert err.max() <= Hn.tol(w)
