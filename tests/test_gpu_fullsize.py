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


def _check_alignment(w, tr, ids_ref, diff):
    if diff.any():
        return None
    cap = O.capacity(w.T, w.k, w.N, w.cap_num, w.cap_den)
    kept = O.capacity_keep(ids_ref, w.N, cap)
    al = O.align(ids_ref, kept, w.N, w.B)
    assert np.array_equal(tr["route_kept"].cpu().numpy().astype(bool), kept)
    assert np.array_equal(tr["sorted_route_ids"].cpu().numpy(), al["sorted_route_ids"])
    assert np.array_equal(tr["expert_offsets"].cpu().numpy(), al["expert_offsets"])
    assert np.array_equal(tr["block_expert"].cpu().numpy(), al["block_expert"])
    return kept


@pytest.mark.parametrize("name", ["switch_capacity_bf16", "mixtral_bf16", "qwen3moe_bf16"])
def test_full_size_layer(name):
    w = W.ALL[name]
    _say("full size", name)
    d = W.layer_inputs(w, device=DEV)
    out, tr = Hn.run_forward(w, d)
    ids_ref, diff = _check_routing(w, d, tr)
    kept = _check_alignment(w, tr, ids_ref, diff)
    g = torch.Generator().manual_seed(7)
    n = 64 if name == "mixtral_bf16" else 256
    sample = np.sort(torch.randperm(w.T, generator=g)[:n].numpy())
    sample = sample[~diff[sample]]
    if kept is not None:  # include every fully dropped token
        gone = np.nonzero(~kept.reshape(w.T, w.k).any(1))[0]
        sample = np.union1d(sample, gone[:64])
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
    out, tr = Hn.run_forward(w, d)
    ids_ref, diff = _check_routing(w, d, tr)
    kept = _check_alignment(w, tr, ids_ref, diff)
    # expert outputs of every route to 3 sampled experts, against the exact oracle and its bf16-stage model
    ids = tr["topk_ids"].cpu().numpy()
    flat = ids.reshape(-1)
    y = tr["y_route"]
    w13_of, w2_of = Hn.weights_f64(w, d, "w13"), Hn.weights_f64(w, d, "w2")
    h64 = Hn.f64(d["h"])
    for e in (0, 97, 255):
        rs = np.nonzero(flat == e)[0]
        assert rs.size > 0
        x = h64[rs // w.k]
        w13, w2 = w13_of(e), w2_of(e)
        exact = O.swiglu_expert(x, w13, w2)
        emul = O.swiglu_expert(x, w13, w2, stage_round=O.round_bf16)
        Hn.check_ffn_surface(w, Hn.f64(y[torch.from_numpy(rs).to(DEV)]), exact, emul, _say)
    # the shared expert on a token sample, through the identity-mode FFN
    g = torch.Generator().manual_seed(8)
    sample = torch.randperm(w.T, generator=g)[:256].sort().values
    hs = d["h"][sample.to(DEV)].contiguous()
    wsamp = w.with_(T=hs.shape[0])
    cfg = Hn.config(wsamp)
    act = torch.empty(hs.shape[0], w.I, dtype=torch.bfloat16, device=DEV)
    ys = torch.empty(hs.shape[0], w.H, dtype=torch.bfloat16, device=DEV)
    M.moe_expert_ffn(cfg, hs, None, None, d["shared_w13"], d["shared_w2"], d["shared_w13_scale"], d["shared_w2_scale"],
                     act, ys)
    torch.cuda.synchronize()
    s13, s2 = Hn.shared_f64(w, d, "w13"), Hn.shared_f64(w, d, "w2")
    x = Hn.f64(hs)
    Hn.check_ffn_surface(w, Hn.f64(ys), O.swiglu_expert(x, s13, s2), O.swiglu_expert(x, s13, s2, stage_round=O.round_bf16),
                         _say)
