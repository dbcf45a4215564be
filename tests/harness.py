"""Test helpers: workload -> config, device buffers, per-op calls, oracle views.

The GPU side is reached only through the binding (the C ABI); the oracle side
only through ``oracle.moe_oracle`` on host copies of the same input bytes.
"""
from __future__ import annotations

import numpy as np
import torch

import top_routing_expert_router_amd as M
import workloads as W
from oracle import moe_oracle as O


def config(w: W.Workload, **kw) -> M.moe_config:
    w = w.with_(**kw) if kw else w
    return M.make_config(w.T, w.H, w.N, w.k, w.I, w.B, cap_num=w.cap_num, cap_den=w.cap_den,
                         n_shared=w.n_shared, renormalize=w.renormalize, act_dtype=w.act_dtype,
                         expert_dtype=w.expert_dtype, scale_block=w.scale_block, reroute_depth=w.reroute_depth,
                         routing=w.routing)


def f64(t: torch.Tensor) -> np.ndarray:
    """Exact float64 view of a host or device tensor (bf16/fp32 decode exactly)."""
    return t.detach().to("cpu").to(torch.float64).numpy()


def weights_f64(w: W.Workload, d: dict, which: str):
    """Callable e -> float64 expert weight (decoded exactly), for the oracle."""
    t = d[which]
    if w.expert_dtype == W.FP8:
        sc = d[which + "_scale"]

        def get(e, t=t, sc=sc):
            codes = t[e].to("cpu").numpy()
            s = f64(sc[e])
            return O.dequantize_blocks(codes, s, w.scale_block)
        return get
    return lambda e, t=t: f64(t[e])


def shared_f64(w: W.Workload, d: dict, which: str) -> np.ndarray:
    t = d["shared_" + which]
    if w.expert_dtype == W.FP8:
        return O.dequantize_blocks(t.to("cpu").numpy(), f64(d["shared_" + which + "_scale"]), w.scale_block)
    return f64(t)


def to_dev(d: dict, dev: str = "cuda") -> dict:
    return {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}


def route_buffers(w: W.Workload, dev="cuda"):
    return dict(logits=torch.empty(w.T, w.N, dtype=torch.float32, device=dev),
                ids=torch.empty(w.T, w.k, dtype=torch.int32, device=dev),
                gates=torch.empty(w.T, w.k, dtype=torch.float32, device=dev),
                margin=torch.empty(w.T, dtype=torch.float32, device=dev))


def align_buffers(cfg, w: W.Workload, dev="cuda"):
    p_max, n_blocks = M.moe_align_sizes(cfg)
    ws = torch.empty(M.moe_workspace_size(cfg, M.MOE_OP_ALIGN), dtype=torch.uint8, device=dev)
    return dict(kept=torch.empty(w.T * w.k, dtype=torch.uint8, device=dev),
                sorted=torch.full((p_max,), -7, dtype=torch.int32, device=dev),
                blocks=torch.full((n_blocks,), -7, dtype=torch.int32, device=dev),
                offsets=torch.full((w.N + 1,), -7, dtype=torch.int32, device=dev),
                npad=torch.full((1,), -7, dtype=torch.int32, device=dev),
                stats=torch.full((w.N + M.STATS_EXTRA,), -7, dtype=torch.int32, device=dev),
                ws=ws)


def run_align(cfg, w, ids_dev, dev="cuda"):
    b = align_buffers(cfg, w, dev)
    M.moe_align(cfg, ids_dev, b["kept"], b["sorted"], b["blocks"], b["offsets"], b["npad"], b["stats"], b["ws"])
    return b


def row_rel_err(got: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """Per row: max |got - ref| / rms(ref row) (rms floored at 1e-30)."""
    rms = np.sqrt(np.mean(ref * ref, axis=1))
    return np.max(np.abs(got - ref), axis=1) / np.maximum(rms, 1e-30)


def tol(w: W.Workload) -> float:
    """Output tolerance, row-RMS relative: 2e-2 for bf16 paths, 1e-4 for fp32."""
    return 1e-4 if w.act_dtype == W.F32 else 2e-2


def topk_valid(logits: np.ndarray, ids: np.ndarray) -> np.ndarray:
    """Per token: are ``ids`` the top-k of ``logits`` under (value desc, lower index first, NaN last)?

    A property check on a result, written without the oracle: distinct ids, listed
    in rank order, and the last selected expert outranks every unselected one.
    """
    T, N = logits.shape
    k = ids.shape[1]
    ok = np.ones(T, dtype=bool)

    def beats(la, a, lb, b):
        na, nb = np.isnan(la), np.isnan(lb)
        if na or nb:
            return (a < b) if (na and nb) else bool(nb)
        if la != lb:
            return la > lb
        return a < b

    for t in range(T):
        row, sel = logits[t], [int(x) for x in ids[t]]
        if len(set(sel)) != k or min(sel) < 0 or max(sel) >= N:
            ok[t] = False
            continue
        if not all(beats(row[a], a, row[b], b) for a, b in zip(sel, sel[1:])):
            ok[t] = False
            continue
        last = sel[-1]
        rest = [e for e in range(N) if e not in sel]
        ok[t] = all(beats(row[last], last, row[e], e) for e in rest)
    return ok


def check_ffn_surface(w: W.Workload, got: np.ndarray, exact: np.ndarray, emul, say=print) -> None:
    """Check an expert-output surface (rows) against the exact fp64 oracle.

    fp32 pipelines: row error <= 1e-4.  bf16 pipelines store the (dequantised)
    weights, act and y in bf16; ``emul`` is the oracle's bf16-stage model of that on
    the same inputs.  The GPU must stay within max(2e-2, 1.25 x the model's own
    error), and nearly every element must lie within 2 bf16 ulps of the model
    (what remains are rounding-boundary flips from fp32 vs fp64 accumulation).
    """
    err = row_rel_err(got, exact)
    if w.act_dtype == W.F32:
        say(f"  max row err {err.max():.3e}")
        assert err.max() <= tol(w), err.max()
        return
    err_model = row_rel_err(emul, exact)
    ulp = np.ldexp(1.0, np.frexp(np.abs(emul))[1] - 8)
    far = np.abs(got - emul) > 2 * ulp + 1e-3 * np.sqrt(np.mean(exact ** 2, axis=1, keepdims=True))
    say(f"  max row err vs exact {err.max():.3e} (bf16-stage model itself {err_model.max():.3e}); "
        f"elements beyond 2 ulp of the model: {far.mean():.2e}")
    assert err.max() <= max(tol(w), 1.25 * err_model.max()), err.max()
    assert far.mean() <= 1e-3, far.mean()


WEIGHT_KEYS = ("w_gate", "w13", "w2", "w13_scale", "w2_scale", "shared_w13", "shared_w2", "shared_w13_scale",
               "shared_w2_scale")


def forward_trace_buffers(cfg, w: W.Workload, T: int = None, dev: str = "cuda") -> dict:
    T = w.T if T is None else T
    p_max, n_blocks = M.moe_align_sizes(cfg)
    act_t = torch.float32 if w.act_dtype == W.F32 else torch.bfloat16
    return dict(logits=torch.empty(T, w.N, device=dev), topk_ids=torch.empty(T, w.k, dtype=torch.int32, device=dev),
                topk_gates=torch.empty(T, w.k, device=dev), margin=torch.empty(T, device=dev),
                route_kept=torch.empty(T * w.k, dtype=torch.uint8, device=dev),
                sorted_route_ids=torch.empty(p_max, dtype=torch.int32, device=dev),
                block_expert=torch.empty(n_blocks, dtype=torch.int32, device=dev),
                expert_offsets=torch.empty(w.N + 1, dtype=torch.int32, device=dev),
                num_padded=torch.empty(1, dtype=torch.int32, device=dev),
                stats=torch.empty(w.N + M.STATS_EXTRA, dtype=torch.int32, device=dev),
                y_route=torch.empty(T * w.k, w.H, dtype=act_t, device=dev))


def run_forward(w: W.Workload, dv: dict, h=None, trace: bool = True, ws=None, dev: str = "cuda"):
    """moe_forward on device inputs ``dv`` (h overridable); returns (out, trace dict)."""
    h = dv["h"] if h is None else h
    T = h.shape[0]
    wT = w.with_(T=T)
    cfg = config(wT)
    act_t = torch.float32 if w.act_dtype == W.F32 else torch.bfloat16
    need = M.moe_workspace_size(cfg, M.MOE_OP_FORWARD)
    if ws is None or ws.numel() < need:
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
    out = torch.empty(T, w.H, dtype=act_t, device=dev)
    tr = forward_trace_buffers(cfg, wT, T, dev) if trace else None
    wts = {k: dv.get(k) for k in WEIGHT_KEYS}
    wts["logit_bias"] = None if dv.get("bias") is None else dv["bias"].to(dev)
    M.moe_forward(cfg, wts, h, h, out, tr, ws)
    torch.cuda.synchronize()
    return out, tr
