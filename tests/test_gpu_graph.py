"""The whole layer inside a HIP graph.

moe_forward allocates nothing, synchronises nothing and records no memset (the GEMMs'
tile counters are cleared by the alignment kernel), so a caller can capture it once and
replay it, the way a serving loop with small, launch-bound batches would.  Each replay
must give the bits of an eager forward on the same inputs; the inputs change between
replays (eager work in between), and every replay is checked.
"""
import sys

import pytest
import torch

import harness as Hn
import top_routing_expert_router_amd as M
import workloads as W

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


CASES = {
    "toy_fp32": W.TOY_FP32,
    "mixtral_bf16_decode": W.MIXTRAL_BF16.with_(T=16),
    "mixtral_bf16": W.MIXTRAL_BF16.with_(T=512),
    "switch_reroute_bf16": W.SWITCH_BF16.with_(T=600, reroute_depth=1),
    "mixtral_ec_bf16": W.MIXTRAL_EC_BF16.with_(T=256),
    "deepseekv3_fp8": W.DEEPSEEKV3_FP8.with_(T=64, N=24, H=1024, I=512),
}


def _bits(t):
    return t.view(torch.int16 if t.element_size() == 2 else torch.int32)


@pytest.mark.parametrize("name", list(CASES))
def test_forward_in_a_graph(name):
    w = CASES[name]
    _say("graph capture", name)
    d = W.layer_inputs(w)
    dv = Hn.to_dev(d)
    cfg = Hn.config(w)
    wts = {k: dv.get(k) for k in Hn.WEIGHT_KEYS}
    wts["logit_bias"] = None if dv.get("bias") is None else dv["bias"].to(DEV)
    ws = torch.empty(M.moe_workspace_size(cfg, M.MOE_OP_FORWARD), dtype=torch.uint8, device=DEV)
    h = dv["h"].clone()
    out_g = torch.empty_like(h)
    out_e = torch.empty_like(h)
    ws_e = torch.empty_like(ws)
    # warm up on the capture's side stream, then capture one forward
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        M.moe_forward(cfg, wts, h, h, out_g, None, ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        M.moe_forward(cfg, wts, h, h, out_g, None, ws)
    gen = torch.Generator(device=DEV).manual_seed(11)
    for rep in range(3):
        # new inputs in place (eager work between replays), the eager reference, then a replay
        h.copy_(dv["h"][torch.randperm(h.shape[0], generator=gen, device=DEV)]
                if rep else dv["h"])
        M.moe_forward(cfg, wts, h, h, out_e, None, ws_e)
        out_g.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(_bits(out_g), _bits(out_e)), (name, rep)
    _say(f"  3 replays bitwise equal to eager")


def test_graph_replay_latency_small_batch():
    """Reported, not asserted against a bound: a decode-sized Mixtral-shaped batch eager
    and as a graph replay."""
    w = W.MIXTRAL_BF16.with_(T=16)
    d = W.layer_inputs(w)
    dv = Hn.to_dev(d)
    cfg = Hn.config(w)
    wts = {k: dv.get(k) for k in Hn.WEIGHT_KEYS}
    ws = torch.empty(M.moe_workspace_size(cfg, M.MOE_OP_FORWARD), dtype=torch.uint8, device=DEV)
    h = dv["h"]
    out = torch.empty_like(h)
    f = lambda: M.moe_forward(cfg, wts, h, h, out, None, ws)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        f()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        f()
    res = {}
    for label, fn in (("eager", f), ("graph", g.replay)):
        for _ in range(5):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(50):
            fn()
        b.record()
        torch.cuda.synchronize()
        res[label] = a.elapsed_time(b) / 50 * 1e3
    _say(f"  T=16 Mixtral-shaped layer: eager {res['eager']:.1f} us, graph replay {res['graph']:.1f} us")
    assert res["graph"] > 0 and res["eager"] > 0
