"""moe_forward_noalloc (no workspace, static per-GPU scratch) against moe_forward.

Through the C ABI on the GPU: two calls in a row, the second with a smaller batch, each
bitwise equal to moe_forward on the same inputs (same kernels, same arithmetic); a config
whose forward needs more than the scratch is refused before anything is enqueued.
"""
import sys

import numpy as np
import pytest
import torch

import top_routing_expert_router_amd as M
import workloads as W
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


def _bits(t):
    return t.view(torch.int16 if t.element_size() == 2 else torch.int32)


@pytest.mark.parametrize("name,T1,T2", [("mixtral_bf16", 1024, 300), ("deepseekv3_fp8", 400, 37),
                                        ("switch_capacity_bf16", 2048, 700), ("toy_fp32", 64, 9)])
def test_noalloc_forward_matches_forward(name, T1, T2):
    w = W.ALL[name]
    _say("noalloc forward", name, T1, T2)
    d = W.layer_inputs(w.with_(T=T1), device=DEV)
    wts = {k: d.get(k) for k in Hn.WEIGHT_KEYS}
    wts["logit_bias"] = None if d.get("bias") is None else d["bias"].to(DEV)  # drawn on the host
    act_t = torch.float32 if w.act_dtype == W.F32 else torch.bfloat16
    for T in (T1, T2):  # two calls in a row, the second smaller
        cfg = Hn.config(w, T=T)
        h = d["h"][:T].contiguous()
        ref = torch.empty(T, w.H, dtype=act_t, device=DEV)
        ws = torch.empty(M.moe_workspace_size(cfg, M.MOE_OP_FORWARD), dtype=torch.uint8, device=DEV)
        ids_ref = torch.empty(T, w.k, dtype=torch.int32, device=DEV)
        M.moe_forward(cfg, wts, h, h, ref, {"topk_ids": ids_ref}, ws)
        out = torch.full((T, w.H), 7.0, dtype=act_t, device=DEV)
        ids = torch.full((T, w.k), -5, dtype=torch.int32, device=DEV)
        M.moe_forward_noalloc(cfg, wts, h, h, out, {"topk_ids": ids})
        torch.cuda.synchronize()
        assert torch.equal(ids, ids_ref)
        assert torch.equal(_bits(out), _bits(ref)), (name, T)
        _say(f"  T={T}: output and ids bitwise equal to moe_forward")


def test_noalloc_rejects_configs_beyond_the_scratch():
    cfg = Hn.config(W.MIXTRAL_BF16)  # T = 4096 needs ~330 MB
    assert M.moe_workspace_size(cfg, M.MOE_OP_FORWARD) > M.NOALLOC_SCRATCH_BYTES
    out = torch.full((8, 8), 3.0, device=DEV)
    with pytest.raises(M.MoeError) as e:
        M.moe_forward_noalloc(cfg, {"w_gate": out, "w13": out, "w2": out}, out, out, out)
    assert e.value.name == "MOE_ERR_WORKSPACE_TOO_SMALL"
    torch.cuda.synchronize()
    assert torch.all(out == 3.0)
