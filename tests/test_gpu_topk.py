"""Top-k at every lane-group size.

A token's experts are ranked by one group of L lanes holding up to 8 experts each:
L = 8 up to 64 experts, 16 up to 128, 32 up to 256.  Routing from given fp32 logits is
checked against the oracle for expert counts on both sides of each group boundary,
with and without renormalisation (ids exact, gates within 1e-6, margin within
1e-6 x max|l|).  The router that computes its own logits (16-token kernel up to 128
experts, two 16-token blocks per workgroup above 64, the wide kernel above 128) must
give bit for bit what the standalone top-k gives on those logits.
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


# (N, k): each side of the 8/16/32-lane boundaries, odd counts that leave lanes empty
COUNTS = [(2, 1), (9, 2), (16, 1), (63, 8), (64, 8), (65, 6), (100, 8), (127, 8), (128, 8), (129, 8),
          (200, 4), (255, 8), (256, 8)]


@pytest.mark.parametrize("renorm", [1, 0])
@pytest.mark.parametrize("N,k", COUNTS, ids=[f"N{n}k{k}" for n, k in COUNTS])
def test_route_from_logits_expert_counts(N, k, renorm):
    T = 517  # not a multiple of any tokens-per-workgroup count
    w = W.DEEPSEEKV3_FP8.with_(T=T, N=N, k=k, renormalize=renorm, near_tie_frac=0.05)
    lg = W.drawn_logits(w, T)
    _say("route_from_logits", N, k, "renormalize", renorm)
    b = Hn.route_buffers(w)
    b["logits"].copy_(lg)
    M.moe_route(Hn.config(w), None, None, None, b["logits"], b["ids"], b["gates"], b["margin"],
                flags=M.MOE_ROUTE_LOGITS_IN)
    torch.cuda.synchronize()
    l64 = lg.double().numpy()
    ids, gates, margin = O.topk_route(l64, k, renormalize=bool(renorm))
    got = b["ids"].cpu().numpy()
    assert np.array_equal(got, ids), np.argwhere(got != ids)[:5]
    gg = b["gates"].cpu().double().numpy()
    assert np.max(np.abs(gg - gates)) <= 1e-6
    if k < N:
        gm = b["margin"].cpu().double().numpy()
        scale = np.max(np.abs(l64), axis=1)
        assert np.all(np.abs(gm - margin) <= 1e-6 * np.maximum(scale, 1.0))


# each router kernel's top-k case: 16-token kernel with 1 to 8 column blocks of 16 experts
# (8 lanes per token and 1, 2, 4 or 8 experts per lane up to 64 experts, 16 lanes above),
# and the wide kernel above 128
@pytest.mark.parametrize("renorm", [1, 0])
@pytest.mark.parametrize("N", [8, 16, 24, 40, 64, 65, 100, 128, 129, 256])
def test_fused_topk_matches_standalone(N, renorm):
    w = W.QWEN3MOE_BF16.with_(T=300, N=N, k=8, renormalize=renorm)
    _say("fused vs standalone top-k", N, "renormalize", renorm)
    h = W.hidden_states(w, device=DEV)
    wg = W.router_weight(w, device=DEV)
    cfg = Hn.config(w)
    a = Hn.route_buffers(w)
    M.moe_route(cfg, h, wg, None, a["logits"], a["ids"], a["gates"], a["margin"])
    b = Hn.route_buffers(w)
    b["logits"].copy_(a["logits"])
    M.moe_route(cfg, None, None, None, b["logits"], b["ids"], b["gates"], b["margin"], flags=M.MOE_ROUTE_LOGITS_IN)
    torch.cuda.synchronize()
    assert torch.equal(a["ids"], b["ids"])
    assert torch.equal(a["gates"].view(torch.int32), b["gates"].view(torch.int32))
    assert torch.equal(a["margin"].view(torch.int32), b["margin"].view(torch.int32))
    # and the routes are a valid top-k of those logits
    assert Hn.topk_valid(a["logits"].cpu().double().numpy(), a["ids"].cpu().numpy()).all()


@pytest.mark.parametrize("N", [64, 100, 128, 200, 256])
def test_router_bias_many_experts(N):
    """The additive per-expert bias on the projection paths for more than 16 experts (the
    16-token kernel with one or two column blocks, the wide kernel above 128): logits within
    1e-5 x max|l| of the oracle, routes exact away from near ties, and the fused top-k bit
    for bit against the standalone top-k on the biased logits."""
    w = W.QWEN3MOE_BF16.with_(T=300, N=N, k=8, zipf_s=0.3)
    _say("router with bias", N)
    h = W.hidden_states(w, device=DEV)
    wg = W.router_weight(w, device=DEV)
    bias = W.logit_bias(w).to(DEV)
    cfg = Hn.config(w)
    a = Hn.route_buffers(w)
    M.moe_route(cfg, h, wg, bias, a["logits"], a["ids"], a["gates"], a["margin"])
    torch.cuda.synchronize()
    l_ref = O.router_logits(Hn.f64(h), Hn.f64(wg), Hn.f64(bias))
    l_gpu = a["logits"].cpu().double().numpy()
    scale = np.max(np.abs(l_ref), axis=1)
    assert (np.max(np.abs(l_gpu - l_ref), axis=1) / scale).max() <= 1e-5
    ids_ref, _, margin_ref = O.topk_route(l_ref, w.k)
    diff = np.any(a["ids"].cpu().numpy() != ids_ref, axis=1)
    assert not np.any(diff & ~(margin_ref <= 2e-5 * scale))
    b = Hn.route_buffers(w)
    b["logits"].copy_(a["logits"])
    M.moe_route(cfg, None, None, None, b["logits"], b["ids"], b["gates"], b["margin"], flags=M.MOE_ROUTE_LOGITS_IN)
    torch.cuda.synchronize()
    assert torch.equal(a["ids"], b["ids"])
    assert torch.equal(a["gates"].view(torch.int32), b["gates"].view(torch.int32))
