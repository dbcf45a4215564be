"""Reroute overflow policy on the GPU, against the oracle.

"Mixture-of-Experts Routing at Inference Time", "The hard part", Figure 2 (an expert
at capacity: drop, or reroute to the 2nd-choice expert) and the mitigation paragraph
after the routing-stats probe.  The decisions (which expert each route runs, which
routes are kept) are integer work: bit-exact against oracle.capacity_reroute on the
GPU's own fp32 logits, and so are the alignment and the stats built on them.  The
layer output with rerouting matches the oracle's forward within the layer tolerance.
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


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    M.lib()


def _reroute_buffers(cfg, w):
    b = Hn.align_buffers(cfg, w)
    b["expert"] = torch.full((w.T * w.k,), -7, dtype=torch.int32, device=DEV)
    return b


def _check_against_oracle(w, ids, logits, depth):
    """moe_align_reroute on (ids, logits) vs the oracle's policy + alignment + stats, bit for bit."""
    cfg = Hn.config(w, reroute_depth=depth)
    b = _reroute_buffers(cfg, w)
    M.moe_align_reroute(cfg, ids.to(DEV), logits.to(DEV), b["expert"], b["kept"], b["sorted"], b["blocks"],
                        b["offsets"], b["npad"], b["stats"], b["ws"])
    torch.cuda.synchronize()
    ids_np = ids.numpy().reshape(w.T, w.k).astype(np.int64)
    cap = O.capacity(w.T, w.k, w.N, w.cap_num, w.cap_den)
    expert, kept, rerouted = O.capacity_reroute(ids_np, logits.double().numpy(), w.N, cap, depth)
    got_e = b["expert"].cpu().numpy()
    assert np.array_equal(got_e, expert), np.argwhere(got_e != expert)[:5]
    assert np.array_equal(b["kept"].cpu().numpy().astype(bool), kept)
    run = np.where(kept, expert, 0).reshape(w.T, w.k)
    al = O.align(run, kept, w.N, w.B)
    for key, name in (("sorted", "sorted_route_ids"), ("offsets", "expert_offsets"), ("blocks", "block_expert")):
        assert np.array_equal(b[key].cpu().numpy(), al[name]), key
    assert int(b["npad"].item()) == al["num_padded"]
    st = b["stats"].cpu().numpy()
    valid = (ids_np >= 0) & (ids_np < w.N)
    load = np.bincount(ids_np[valid], minlength=w.N)
    assert np.array_equal(st[:w.N], load)
    N = w.N
    assert st[N + M.STAT["kept"]] == kept.sum()
    assert st[N + M.STAT["rerouted"]] == rerouted.sum()
    assert st[N + M.STAT["dropped"]] == (valid.reshape(-1) & ~kept).sum()
    assert st[N + M.STAT["invalid"]] == (~valid).sum()
    assert st[N + M.STAT["capacity"]] == (-1 if cap is None else cap)
    assert st[N + M.STAT["num_padded"]] == al["num_padded"]
    assert st[N + M.STAT["unpicked"]] == 0 and st[N + M.STAT["max_picks"]] == 0
    return kept.sum(), rerouted.sum()


@pytest.mark.parametrize("depth", [0, 1, 3, 15])
def test_switch_reroute_bit_exact(depth):
    """The capacity workload (2048 tokens, 16 experts, top-1, cf 5/4, Zipf-skewed logits)."""
    w = W.SWITCH_BF16
    d, dv = inputs(w)
    cfg = Hn.config(w)
    r = Hn.route_buffers(w)
    M.moe_route(cfg, dv["h"], dv["w_gate"], dv["bias"], r["logits"], r["ids"], r["gates"], r["margin"])
    torch.cuda.synchronize()
    kept, rer = _check_against_oracle(w, r["ids"].cpu(), r["logits"].cpu(), depth)
    _say(f"switch reroute depth {depth}: kept {kept} of {w.T}, rerouted {rer}")
    if depth:
        assert rer > 0
    if depth == 0:  # equals the drop policy of moe_align
        b = Hn.align_buffers(cfg, w)
        M.moe_align(cfg, r["ids"], b["kept"], b["sorted"], b["blocks"], b["offsets"], b["npad"], b["stats"], b["ws"])
        torch.cuda.synchronize()
        b2 = _reroute_buffers(cfg, w)
        M.moe_align_reroute(cfg, r["ids"], r["logits"], b2["expert"], b2["kept"], b2["sorted"], b2["blocks"],
                            b2["offsets"], b2["npad"], b2["stats"], b2["ws"])
        torch.cuda.synchronize()
        for key in ("kept", "sorted", "blocks", "offsets", "npad", "stats"):
            assert torch.equal(b[key], b2[key]), key


CASES = [
    # (T, N, k, cap_num, cap_den, depth, invalid fraction, seed)
    (3000, 8, 2, 1, 2, 6, 0.0, 1),      # tight capacity, top-2, whole ranking
    (3000, 8, 2, 3, 4, 1, 0.02, 2),     # second choice only, some invalid ids
    (777, 64, 6, 1, 3, 10, 0.01, 3),    # many experts, ragged T
    (40000, 128, 8, 9, 10, 4, 0.0, 4),  # large: 320k routes through the one-workgroup pass
    (5, 4, 1, 1, 1, 3, 0.0, 5),         # tiny
    (1, 8, 2, 1, 1, 6, 0.0, 6),         # one token: cap = 0, nothing can be placed
    (1000, 2, 1, 1, 1, 1, 0.0, 7),      # two experts: 2 lanes per token in the ranking kernel
    (2500, 24, 3, 1, 1, 21, 0.01, 8),   # 24 experts (32 lanes per token), whole ranking
    (300, 256, 8, 1, 1, 248, 0.0, 9),   # 256 experts, whole ranking (4 ranks per lane)
]


@pytest.mark.parametrize("case", CASES, ids=[str(c) for c in CASES])
def test_reroute_drawn_logits_and_recorded_ids(case):
    T, N, k, cn, cd, depth, bad, seed = case
    w = W.Workload("reroute_case", T=T, H=128, N=N, k=k, I=128, B=16, act_dtype=W.F32, expert_dtype=W.F32,
                   cap_num=cn, cap_den=cd, seed=seed, near_tie_frac=0.05)
    lg = W.drawn_logits(w, T)
    lg[lg > 1.5] = 1.5  # plateaus: exact ties in the rankings
    ids, _, _ = O.topk_route(lg.double().numpy(), k)
    ids = torch.from_numpy(ids.astype(np.int32))
    _check_against_oracle(w, ids.reshape(-1), lg, depth)
    # recorded ids that are not this run's top-k (replay), some outside [0, N)
    g = torch.Generator().manual_seed(seed)
    rec = torch.argsort(torch.rand(T, N, generator=g), dim=1)[:, :k].to(torch.int32)
    if bad:
        m = torch.rand(T, k, generator=g) < bad
        rec[m] = N
    _check_against_oracle(w, rec.reshape(-1), lg, depth)


def test_forward_with_reroute():
    w = W.SWITCH_REROUTE_BF16.with_(T=600)
    d, dv = inputs(W.SWITCH_BF16.with_(T=600))
    _say("forward with reroute", w.name, w.T)
    out, tr = Hn.run_forward(w, dv)
    res = O.moe_forward(Hn.f64(d["h"]), Hn.f64(d["w_gate"]), Hn.weights_f64(w, d, "w13"), Hn.weights_f64(w, d, "w2"),
                        k=w.k, B=w.B, cap_num=w.cap_num, cap_den=w.cap_den, bias=Hn.f64(d["bias"]),
                        residual=Hn.f64(d["residual"]), reroute_depth=w.reroute_depth)
    ids = tr["topk_ids"].cpu().numpy()
    scale = np.max(np.abs(res["logits"]), axis=1)
    near = res["margin"] <= 2e-5 * scale
    same = np.array_equal(ids, res["ids"])
    _say(f"  routes equal {same}, near-tie tokens {near.sum()}, rerouted {res['stats']['rerouted']}")
    assert res["stats"]["rerouted"] > 0
    if same:  # the whole decision chain is integer work on equal ids and equal rankings
        assert np.array_equal(tr["route_kept"].cpu().numpy().astype(bool), res["kept"])
        assert np.array_equal(tr["sorted_route_ids"].cpu().numpy(), res["align"]["sorted_route_ids"])
        err = Hn.row_rel_err(Hn.f64(out), res["out"])
        _say(f"  max out row err {err.max():.3e}")
        assert err.max() <= Hn.tol(w)
    else:
        assert np.all(np.any(ids != res["ids"], axis=1) <= near)
