"""Router replay and route-trace export on the GPU.

Replay ("Mixture-of-experts routing & LLM repeatability", router replay paragraph):
recorded expert ids of an earlier run are used again, so the expert path is fixed;
the gates still come from this run's scores.  Checked here:
  - replaying a run's own ids reproduces its routing outputs and its layer output
    bit for bit (moe_route with MOE_ROUTE_IDS_IN, moe_forward_replay);
  - replaying other recorded ids (including ids outside [0, N)) gives the oracle's
    replay gates on the GPU's own logits, and the layer output of the oracle's
    forward with the same recorded ids;
  - the trace a forward exports (logits, ids, gates, margin, alignment, y rows)
    equals what the standalone entry points compute from the same inputs, bit for
    bit -- the route-trace half of the pages' repeatability checklist ("record
    per-token logits and expert routes").
"""
import numpy as np
import pytest
import torch

import top_routing_expert_router_amd as M
import workloads as W
from oracle import moe_oracle as O
from tests import harness as Hn
from tests.test_gpu_parity import SMALL, inputs, _say

pytestmark = pytest.mark.gpu
DEV = "cuda"
NAMES = ["toy_fp32", "switch_capacity_bf16", "mixtral_bf16", "qwen3moe_bf16", "deepseekv3_fp8"]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    M.lib()


def _bits(t):
    return t.contiguous().view(torch.int32) if t.dtype == torch.float32 else t.contiguous().view(torch.int16)


def _route(w, dv, flags=0, ids=None, logits=None):
    cfg = Hn.config(w)
    b = Hn.route_buffers(w)
    if ids is not None:
        b["ids"].copy_(ids)
    if logits is not None:
        b["logits"].copy_(logits)
    M.moe_route(cfg, dv["h"], dv["w_gate"], dv.get("bias"), b["logits"], b["ids"], b["gates"], b["margin"],
                flags=flags)
    torch.cuda.synchronize()
    return b


def _recorded_ids(w, seed, invalid_frac=0.0):
    """Distinct expert ids per token in a seeded order; a fraction replaced by ids outside [0, N)."""
    g = torch.Generator().manual_seed(seed)
    ids = torch.argsort(torch.rand(w.T, w.N, generator=g), dim=1)[:, :w.k].to(torch.int32)
    if invalid_frac:
        bad = torch.rand(w.T, w.k, generator=g) < invalid_frac
        ids[bad] = torch.where(torch.rand(int(bad.sum()), generator=g) < 0.5, -1, w.N).to(torch.int32)
    return ids


@pytest.mark.parametrize("renorm", [1, 0])
@pytest.mark.parametrize("name", NAMES)
def test_route_replay_of_own_ids_is_bitwise(name, renorm):
    w = SMALL[name].with_(renormalize=renorm)
    d, dv = inputs(SMALL[name])
    _say("route replay (own ids)", name, "renormalize", renorm)
    ref = _route(w, dv)
    rec = ref["ids"].clone()
    for flags, lg in ((M.MOE_ROUTE_IDS_IN, None), (M.MOE_ROUTE_IDS_IN | M.MOE_ROUTE_LOGITS_IN, ref["logits"])):
        got = _route(w, dv, flags=flags, ids=rec, logits=lg)
        assert torch.equal(got["ids"], rec)  # the recorded ids are only read
        assert torch.equal(_bits(got["logits"]), _bits(ref["logits"]))
        assert torch.equal(_bits(got["gates"]), _bits(ref["gates"]))
        assert torch.equal(_bits(got["margin"]), _bits(ref["margin"]))


@pytest.mark.parametrize("renorm", [1, 0])
@pytest.mark.parametrize("name", NAMES)
def test_route_replay_of_other_ids(name, renorm):
    w = SMALL[name].with_(renormalize=renorm)
    d, dv = inputs(SMALL[name])
    _say("route replay (other ids)", name, "renormalize", renorm)
    ref = _route(w, dv)
    rec = _recorded_ids(w, seed=11, invalid_frac=0.05)
    got = _route(w, dv, flags=M.MOE_ROUTE_IDS_IN | M.MOE_ROUTE_LOGITS_IN, ids=rec, logits=ref["logits"])
    lg = ref["logits"].cpu().double().numpy()
    gates, margin = O.replay_route(lg, rec.numpy(), renormalize=bool(renorm))
    gg = got["gates"].cpu().double().numpy()
    fin = np.isfinite(gates)
    assert np.array_equal(np.isfinite(gg), fin)
    assert np.max(np.abs(gg[fin] - gates[fin])) <= 1e-6
    valid = (rec.numpy() >= 0) & (rec.numpy() < w.N)
    # an id outside [0, N) weighs nothing; renormalising over a token with no valid
    # id divides 0 by 0 (NaN on both sides -- its routes are never kept)
    some = valid.any(axis=1, keepdims=True) if renorm else np.ones((w.T, 1), bool)
    assert np.all(gg[~valid & some] == 0)
    assert np.all(np.isnan(gg[~some.repeat(w.k, axis=1)]))
    # the margin is this run's own, whatever ids are replayed
    assert torch.equal(_bits(got["margin"]), _bits(ref["margin"]))


def _weights(dv):
    wts = {k: dv.get(k) for k in Hn.WEIGHT_KEYS}
    wts["logit_bias"] = dv.get("bias")
    return wts


@pytest.mark.parametrize("name", NAMES)
def test_forward_replay_of_own_ids_is_bitwise(name):
    w = SMALL[name]
    d, dv = inputs(w)
    _say("forward replay (own ids)", name)
    out, tr = Hn.run_forward(w, dv)
    cfg = Hn.config(w)
    ws = torch.empty(M.moe_workspace_size(cfg, M.MOE_OP_FORWARD), dtype=torch.uint8, device=DEV)
    out2 = torch.empty_like(out)
    tr2 = Hn.forward_trace_buffers(cfg, w)
    M.moe_forward_replay(cfg, _weights(dv), dv["h"], dv["h"], tr["topk_ids"], out2, tr2, ws)
    torch.cuda.synchronize()
    assert torch.equal(_bits(out2), _bits(out))
    for key in ("logits", "topk_gates", "margin", "route_kept", "sorted_route_ids", "expert_offsets", "stats"):
        a, b = tr[key], tr2[key]
        assert torch.equal(_bits(a) if a.is_floating_point() else a, _bits(b) if b.is_floating_point() else b), key


@pytest.mark.parametrize("name", NAMES)
def test_forward_replay_of_other_ids(name):
    w = SMALL[name]
    d, dv = inputs(w)
    _say("forward replay (other ids)", name)
    _, tr = Hn.run_forward(w, dv)
    rec = ((tr["topk_ids"].cpu() + 1) % w.N).to(torch.int32)  # a different, still distinct, route per token
    cfg = Hn.config(w)
    ws = torch.empty(M.moe_workspace_size(cfg, M.MOE_OP_FORWARD), dtype=torch.uint8, device=DEV)
    out = torch.empty(w.T, w.H, dtype=torch.float32 if w.act_dtype == W.F32 else torch.bfloat16, device=DEV)
    tr2 = Hn.forward_trace_buffers(cfg, w)
    M.moe_forward_replay(cfg, _weights(dv), dv["h"], dv["h"], rec.to(DEV), out, tr2, ws)
    torch.cuda.synchronize()
    res = O.moe_forward(Hn.f64(d["h"]), Hn.f64(d["w_gate"]), Hn.weights_f64(w, d, "w13"), Hn.weights_f64(w, d, "w2"),
                        k=w.k, B=w.B, cap_num=w.cap_num, cap_den=w.cap_den,
                        bias=None if d["bias"] is None else Hn.f64(d["bias"]), residual=Hn.f64(d["residual"]),
                        shared_w13=Hn.shared_f64(w, d, "w13") if w.n_shared else None,
                        shared_w2=Hn.shared_f64(w, d, "w2") if w.n_shared else None, replay_ids=rec.numpy())
    # capacity and alignment depend only on the ids: bit-exact
    assert np.array_equal(tr2["route_kept"].cpu().numpy().astype(bool), res["kept"])
    assert np.array_equal(tr2["sorted_route_ids"].cpu().numpy(), res["align"]["sorted_route_ids"])
    assert np.array_equal(tr2["expert_offsets"].cpu().numpy(), res["align"]["expert_offsets"])
    gg = tr2["topk_gates"].cpu().double().numpy()
    assert np.max(np.abs(gg - res["gates"])) <= 5e-5  # logits within 1e-5 relative move gates less
    err = Hn.row_rel_err(Hn.f64(out), res["out"])
    _say(f"  max out row err {err.max():.3e}")
    assert err.max() <= Hn.tol(w)


@pytest.mark.parametrize("name", NAMES)
def test_trace_export_matches_standalone_calls(name):
    w = SMALL[name]
    d, dv = inputs(w)
    _say("trace export", name)
    cfg = Hn.config(w)
    act_t = torch.float32 if w.act_dtype == W.F32 else torch.bfloat16
    p_max, _ = M.moe_align_sizes(cfg)
    ws = torch.empty(M.moe_workspace_size(cfg, M.MOE_OP_FORWARD), dtype=torch.uint8, device=DEV)
    tr = Hn.forward_trace_buffers(cfg, w)
    tr["act"] = torch.empty(p_max, w.I, dtype=act_t, device=DEV)
    out = torch.empty(w.T, w.H, dtype=act_t, device=DEV)
    M.moe_forward(cfg, _weights(dv), dv["h"], dv["h"], out, tr, ws)
    torch.cuda.synchronize()
    # the same steps through the standalone entry points
    r = _route(w, dv)
    for a, b in (("logits", "logits"), ("topk_ids", "ids"), ("topk_gates", "gates"), ("margin", "margin")):
        x, y = tr[a], r[b]
        assert torch.equal(_bits(x) if x.is_floating_point() else x, _bits(y) if y.is_floating_point() else y), a
    al = Hn.align_buffers(cfg, w)
    M.moe_align(cfg, r["ids"], al["kept"], al["sorted"], al["blocks"], al["offsets"], al["npad"], al["stats"], al["ws"])
    for a, b in (("route_kept", "kept"), ("sorted_route_ids", "sorted"), ("block_expert", "blocks"),
                 ("expert_offsets", "offsets"), ("num_padded", "npad"), ("stats", "stats")):
        assert torch.equal(tr[a], al[b]), a
    act = torch.empty_like(tr["act"])
    y = torch.empty_like(tr["y_route"])
    # rows of dropped routes and padding are never written: start both from the same bytes
    y.copy_(tr["y_route"])
    act.copy_(tr["act"])
    npad = int(al["npad"].item())
    act[:npad].zero_()
    kept = al["kept"].bool()
    y.index_fill_(0, torch.nonzero(kept).flatten(), 0)
    M.moe_expert_ffn(cfg, dv["h"], al["sorted"], al["offsets"], dv["w13"], dv["w2"], dv.get("w13_scale"),
                     dv.get("w2_scale"), act, None, y)
    torch.cuda.synchronize()
    valid = al["sorted"][:npad] < w.T * w.k
    assert torch.equal(_bits(act[:npad][valid]), _bits(tr["act"][:npad][valid]))
    assert torch.equal(_bits(y[kept]), _bits(tr["y_route"][kept]))
    shared = None
    if w.n_shared:
        sact = torch.empty(w.T, w.I, dtype=act_t, device=DEV)
        shared = torch.empty(w.T, w.H, dtype=act_t, device=DEV)
        M.moe_expert_ffn(cfg, dv["h"], None, None, dv["shared_w13"], dv["shared_w2"], dv.get("shared_w13_scale"),
                         dv.get("shared_w2_scale"), sact, None, shared)
    out2 = torch.empty_like(out)
    M.moe_combine(cfg, y, r["gates"], al["kept"], shared, dv["h"], out2)
    torch.cuda.synchronize()
    assert torch.equal(_bits(out2), _bits(out))
