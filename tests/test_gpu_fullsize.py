"""Parity at the workloads' full sizes, in the launch configuration the benchmark uses.

Routing, capacity and alignment are checked on every token; expert outputs and
layer outputs on seeded samples the oracle computes one by one (all experts of
the sampled tokens, or all routes of a sample of experts when the weights are
too many to decode).
"""
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


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    M.lib()


def _check_routing(w, d, tr):
    l_ref = O.router_logits(Hn.f64(d["h"]), Hn.f64(d["w_gate"]), None if d["bias"] is None else Hn.f64(d["bias"]))
    l_gpu = tr["logits"].cpu().double().numpy()
    scale = np.max(np.abs(l_ref), axis=1)
    assert (np.max(np.abs(l_gpu - l_ref), axis=1) / scale).max() <= 1e-5
    ids_ref, gates_ref, margin_ref = O.topk_route(l_ref, w.k)
    ids = tr["topk_ids"].cpu().numpy()
    diff = np.any(ids != ids_ref, axis=1)
    near = margin_ref <= 2e-5 * scale
    _say(f"  tokens {w.T}: near-tie {near.sum()}, routed differently {diff.sum()} (all near-tie: {not np.any(diff & ~near)})")
    assert not np.any(diff & ~near)
    assert Hn.topk_valid(l_gpu, ids).all()
    return ids_ref, diff


def _check_alignment(w, tr):
    """Oracle capacity and alignment applied to the GPU's own expert ids: bit-exact for every
    route, with no exclusion (a near-tie token routed differently from the fp64 oracle still
    has its capacity and alignment checked, on the ids it got)."""
    ids = tr["topk_ids"].cpu().numpy().astype(np.int64)
    cap = O.capacity(w.T, w.k, w.N, w.cap_num, w.cap_den)
    kept = O.capacity_keep(ids, w.N, cap)
    al = O.align(ids, kept, w.N, w.B)
    assert np.array_equal(tr["route_kept"].cpu().numpy().astype(bool), kept)
    assert np.array_equal(tr["sorted_route_ids"].cpu().numpy(), al["sorted_route_ids"])
    assert np.array_equal(tr["expert_offsets"].cpu().numpy(), al["expert_offsets"])
    assert np.array_equal(tr["block_expert"].cpu().numpy(), al["block_expert"])
    assert int(tr["num_padded"].item()) == al["num_padded"]
    st = O.routing_stats(ids, kept, w.N, cap)
    gs = tr["stats"].cpu().numpy()
    assert np.array_equal(gs[:w.N], st["load"])
    health = M.moe_routing_health_from_stats(Hn.config(w), gs)
    assert health["imbalance_ratio"] == pytest.approx(st["imbalance_ratio"], rel=1e-15)
    assert health["drop_fraction"] == pytest.approx(st["drop_fraction"], rel=1e-15, abs=0)
    assert health["dropped_routes"] == st["dropped_tokens"]
    _say(f"  alignment bit-exact on the GPU's ids; imbalance {health['imbalance_ratio']:.4f}, "
         f"drop fraction {health['drop_fraction']:.4f}")
    return kept


@pytest.mark.parametrize("name", ["switch_capacity_bf16", "mixtral_bf16", "qwen3moe_bf16", "mixtral_bf16@65536"])
def test_full_size_layer(name):
    """The whole layer at a workload's full size (and the Mixtral shape at the largest T the
    ABI accepts): routing, capacity and alignment of every token, outputs on a sample."""
    base, _, t = name.partition("@")
    w = W.ALL[base] if not t else W.ALL[base].with_(T=int(t))
    name = base
    _say("full size", w.name, w.T)
    d = W.layer_inputs(w, device=DEV)
    out, tr = Hn.run_forward(w, d)
    ids_ref, diff = _check_routing(w, d, tr)
    kept = _check_alignment(w, tr)
    g = torch.Generator().manual_seed(7)
    n = 64 if name == "mixtral_bf16" else 256
    sample = np.sort(torch.randperm(w.T, generator=g)[:n].numpy())
    sample = sample[~diff[sample]]
    gone = np.nonzero(~kept.reshape(w.T, w.k).any(1))[0]   # include fully dropped tokens
    sample = np.union1d(sample, gone[~diff[gone]][:64])
    res = O.moe_forward(Hn.f64(d["h"]), Hn.f64(d["w_gate"]), Hn.weights_f64(w, d, "w13"), Hn.weights_f64(w, d, "w2"),
                        k=w.k, B=w.B, cap_num=w.cap_num, cap_den=w.cap_den,
                        bias=None if d["bias"] is None else Hn.f64(d["bias"]), residual=Hn.f64(d["h"]),
                        tokens=sample)
    err = Hn.row_rel_err(Hn.f64(out)[sample], res["out"])
    _say(f"  sampled {sample.size} tokens: max out row err {err.max():.3e}")
    assert err.max() <= Hn.tol(w)


def test_full_size_deepseek_fp8():
    w = W.DEEPSEEKV3_FP8
    _say("full size deepseek fp8")
    d = W.layer_inputs(w, device=DEV)
    cfg = Hn.config(w)
    p_max, _ = M.moe_align_sizes(cfg)
    out, tr = Hn.run_forward(w, d, act=True)
    ids_ref, diff = _check_routing(w, d, tr)
    _check_alignment(w, tr)
    ids = tr["topk_ids"].cpu().numpy()
    flat = ids.reshape(-1)
    sorted_ids = tr["sorted_route_ids"].cpu().numpy()
    # the fast fp8 decode is the oracle's, exactly (one expert compared in full)
    w13_of, w2_of = Hn.weights_f64(w, d, "w13", fast=True), Hn.weights_f64(w, d, "w2", fast=True)
    assert np.array_equal(w2_of(5), Hn.weights_f64(w, d, "w2")(5))
    h64 = Hn.f64(d["h"])
    # every route of 3 experts, surface by surface: activation rows (by padded row) and W2 rows
    rows = np.nonzero(np.isin(flat[np.minimum(sorted_ids, flat.size - 1)], (0, 97, 255)) & (sorted_ids < flat.size))[0]
    routes = sorted_ids[rows]
    Hn.check_expert_rows(w, h64[routes // w.k], flat[routes], w13_of, w2_of,
                         Hn.f64(tr["act"][torch.from_numpy(rows).to(DEV)]),
                         Hn.f64(tr["y_route"][torch.from_numpy(routes).to(DEV)]), say=_say)
    # the layer output, shared expert inside the forward, on a token sample against the exact
    # oracle (each needed expert decoded one at a time); tokens routed differently at a near
    # tie are left out of the sample and reported by _check_routing
    g = torch.Generator().manual_seed(9)
    sample = np.sort(torch.randperm(w.T, generator=g)[:24].numpy())
    sample = sample[~diff[sample]]
    s13 = Hn.weights_f64(w, {"w": d["shared_w13"][None], "w_scale": d["shared_w13_scale"][None]}, "w", fast=True)(0)
    s2 = Hn.weights_f64(w, {"w": d["shared_w2"][None], "w_scale": d["shared_w2_scale"][None]}, "w", fast=True)(0)
    res = O.moe_forward(h64, Hn.f64(d["w_gate"]), w13_of, w2_of, k=w.k, B=w.B, residual=h64, tokens=sample,
                        shared_w13=s13, shared_w2=s2)
    err = Hn.row_rel_err(Hn.f64(out)[sample], res["out"])
    _say(f"  forward output, {sample.size} sampled tokens ({np.unique(flat.reshape(w.T, w.k)[sample]).size} experts "
         f"+ shared): max row err {err.max():.3e} (tol {Hn.tol(w)})")
    assert err.max() <= Hn.tol(w)
    # the shared expert alone on a token sample, through the identity-mode FFN
    g = torch.Generator().manual_seed(8)
    sample = torch.randperm(w.T, generator=g)[:256].sort().values
    hs = d["h"][sample.to(DEV)].contiguous()
    wsamp = w.with_(T=hs.shape[0])
    cfg = Hn.config(wsamp)
    act = torch.empty(hs.shape[0], w.I, dtype=torch.bfloat16, device=DEV)
    ys = torch.empty(hs.shape[0], w.H, dtype=torch.bfloat16, device=DEV)
    M.moe_expert_ffn(cfg, hs, None, None, d["shared_w13"], d["shared_w2"], d["shared_w13_scale"], d["shared_w2_scale"],
                     act, None, ys)
    torch.cuda.synchronize()
    Hn.check_expert_rows(w, Hn.f64(hs), np.zeros(hs.shape[0], np.int64), lambda e: s13, lambda e: s2, Hn.f64(act),
                         Hn.f64(ys), say=_say)
