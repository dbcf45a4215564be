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


def weights_f64(w: W.Workload, d: dict, which: str, fast: bool = False):
    """Callable e -> float64 expert weight (decoded exactly), for the oracle.

    fp8: O.dequantize_blocks; with ``fast``, the same values from torch's E4M3FN decode (every
    code pinned equal to the oracle's decode) times the block scale in float64, computed where
    the codes live -- exact either way, one expert at a time."""
    t = d[which]
    if w.expert_dtype == W.FP8:
        sc = d[which + "_scale"]

        def get(e, t=t, sc=sc):
            codes = t[e].to("cpu").numpy()
            s = f64(sc[e])
            return O.dequantize_blocks(codes, s, w.scale_block)

        def get_fast(e, t=t, sc=sc):
            b = w.scale_block
            q = t[e].view(torch.float8_e4m3fn).to(torch.float64)
            s = sc[e].to(torch.float64).repeat_interleave(b, 0).repeat_interleave(b, 1)
            return (q * s).cpu().numpy()
        return get_fast if fast else get
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


# ---- expert surfaces, element by element, each from the surface before it
#
# The expert path has three stored surfaces ("Route-Block Membership Selects Packed-AWQ
# Arithmetic", "The boundary that mattered"): the W13 output, the activation and the W2
# output.  Each is checked against the exact (fp64) value of its own step computed from the
# operands the GPU multiplies -- h rows and the weights for W13 and the activation, the GPU's
# stored activation for W2 -- with a worst-case bound that follows from the arithmetic:
#   - bf16 x bf16 products are exact in fp32; an fp32 sum of K of them, in any order and
#     whatever the rounding of each addition, is off by at most gamma_K * sum |a_i w_i|,
#     gamma_K = K u / (1 - K u) with u = 2^-23 (covers round-to-nearest and truncation);
#   - a store in the act dtype rounds once: 2^-8 relative in bf16, exact in fp32;
#   - fp8 weights are decoded exactly, scaled by their block's bf16 scale in fp32 (exact:
#     4 + 8 significant bits) and rounded to bf16 before the product, so the weight the GPU
#     multiplies is round_bf16(e4m3(q) * s);
#   - silu on the GPU (hardware exp and reciprocal, or expf and division on the fp32 path)
#     is within 2^-18 relative of silu, plus 1e-30 absolute where e^-x overflows.
# A wrong row, column, weight block, scale or transposed operand moves an element by about
# its own size, far outside these bounds (about 1% of the row's scale at K = 4096).

ACC_U = 2.0 ** -23
SILU_REL = 2.0 ** -18


def gamma(K: int) -> float:
    return K * ACC_U / (1.0 - K * ACC_U)


def store_rel(w: W.Workload) -> float:
    """Relative rounding of one store in the act dtype."""
    return 0.0 if w.act_dtype == W.F32 else 2.0 ** -8


def effective_weights(w: W.Workload, w_of):
    """Callable e -> the weight the GPU multiplies: as stored (bf16, fp32), or for fp8 the
    block-scaled decode rounded to bf16."""
    if w.expert_dtype == W.FP8:
        return lambda e: O.round_bf16(w_of(e))
    return w_of


def check_product_surface(w: W.Workload, got: np.ndarray, a: np.ndarray, wt: np.ndarray) -> float:
    """got ~= a @ wt.T, stored in the act dtype after an fp32 accumulation over K = a.shape[1].
    Asserts every element is within the bound; returns max |err| / bound (how tight it is)."""
    exact = a @ wt.T
    S = np.abs(a) @ np.abs(wt).T
    r = store_rel(w)
    bound = r * np.abs(exact) + (1.0 + r) * gamma(a.shape[1]) * S
    err = np.abs(got - exact)
    bad = err > bound
    assert not bad.any(), (np.argwhere(bad)[:5], err[bad][:5], bound[bad][:5])
    return float((err / np.maximum(bound, 1e-300)).max())


def check_activation_surface(w: W.Workload, got: np.ndarray, x: np.ndarray, w13: np.ndarray) -> float:
    """got ~= silu(x W1^T) * (x W3^T) (the activation), from fp32 gate and up accumulations
    over K = x.shape[1], silu, an fp32 product and one store in the act dtype."""
    I = w13.shape[0] // 2
    u = O.w13_projection(x, w13)
    g = gamma(x.shape[1])
    S = np.abs(x) @ np.abs(w13).T
    du, dv = g * S[:, :I], g * S[:, I:]
    up = u[:, I:]
    s = O.silu(u[:, :I])
    exact = O.swiglu_activation(x, w13)
    # |silu'| <= 1.1, so the gate's accumulation error moves silu by at most 1.1 du
    pre = 1.1 * du * (np.abs(up) + dv) + np.abs(s) * dv
    mag = (np.abs(s) + 1.1 * du) * (np.abs(up) + dv)
    rel = (1.0 + SILU_REL) * (1.0 + 2.0 ** -24) * (1.0 + store_rel(w)) - 1.0
    bound = pre + rel * mag + 1e-30
    err = np.abs(got - exact)
    bad = err > bound
    assert not bad.any(), (np.argwhere(bad)[:5], err[bad][:5], bound[bad][:5])
    return float((err / bound).max())


def check_expert_rows(w: W.Workload, x_rows: np.ndarray, experts: np.ndarray, w13_of, w2_of,
                      got_act: np.ndarray, got_y: np.ndarray, got_w13=None, say=print) -> None:
    """Row i ran expert experts[i] on input row x_rows[i]: its W13 output (if given), activation
    and W2 output are checked surface by surface (bounds above); the W2 check starts from the
    GPU's own stored activation.  w13_of / w2_of give the exact fp64 weights."""
    e13, e2 = effective_weights(w, w13_of), effective_weights(w, w2_of)
    worst = {"W13": 0.0, "act": 0.0, "W2": 0.0}
    for e in np.unique(experts):
        idx = np.nonzero(experts == e)[0]
        x = x_rows[idx]
        W13 = e13(int(e))
        if got_w13 is not None:
            worst["W13"] = max(worst["W13"], check_product_surface(w, got_w13[idx], x, W13))
        worst["act"] = max(worst["act"], check_activation_surface(w, got_act[idx], x, W13))
        worst["W2"] = max(worst["W2"], check_product_surface(w, got_y[idx], got_act[idx], e2(int(e))))
    say(f"  {x_rows.shape[0]} rows, {np.unique(experts).size} experts: max |err| / bound "
        + ", ".join(f"{k} {v:.3f}" for k, v in worst.items() if got_w13 is not None or k != "W13"))


WEIGHT_KEYS = ("w_gate", "w13", "w2", "w13_scale", "w2_scale", "shared_w13", "shared_w2", "shared_w13_scale",
               "shared_w2_scale")


def forward_trace_buffers(cfg, w: W.Workload, T: int = None, dev: str = "cuda", act: bool = False) -> dict:
    T = w.T if T is None else T
    p_max, n_blocks = M.moe_align_sizes(cfg)
    act_t = torch.float32 if w.act_dtype == W.F32 else torch.bfloat16
    extra = {"act": torch.empty(p_max, w.I, dtype=act_t, device=dev)} if act else {}
    return dict(**extra, logits=torch.empty(T, w.N, device=dev), topk_ids=torch.empty(T, w.k, dtype=torch.int32, device=dev),
                topk_gates=torch.empty(T, w.k, device=dev), margin=torch.empty(T, device=dev),
                route_kept=torch.empty(T * w.k, dtype=torch.uint8, device=dev),
                sorted_route_ids=torch.empty(p_max, dtype=torch.int32, device=dev),
                block_expert=torch.empty(n_blocks, dtype=torch.int32, device=dev),
                expert_offsets=torch.empty(w.N + 1, dtype=torch.int32, device=dev),
                num_padded=torch.empty(1, dtype=torch.int32, device=dev),
                stats=torch.empty(w.N + M.STATS_EXTRA, dtype=torch.int32, device=dev),
                y_route=torch.empty(T * w.k, w.H, dtype=act_t, device=dev))


def run_forward(w: W.Workload, dv: dict, h=None, trace: bool = True, ws=None, dev: str = "cuda", act: bool = False):
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
    tr = forward_trace_buffers(cfg, wT, T, dev, act=act) if trace else None
    wts = {k: dv.get(k) for k in WEIGHT_KEYS}
    wts["logit_bias"] = None if dv.get("bias") is None else dv["bias"].to(dev)
    M.moe_forward(cfg, wts, h, h, out, tr, ws)
    torch.cuda.synchronize()
    return out, tr
