"""Python binding of libmoe_mi355x.so (the C ABI in include/moe.h).

Argument marshalling only: every step of the layer runs in the HIP library.
Functions carry the C entry points' names and take torch tensors (device
memory), None for NULL, and an optional stream (default: torch's current
stream).  A non-OK status raises MoeError.  Importing the package loads the
shared library and fails loudly if it has not been built.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

from .build import LIB_PATH

__all__ = [
    "MoeError", "moe_config", "moe_weights", "moe_trace", "make_config", "lib",
    "moe_abi_version", "moe_status_str", "moe_validate_config", "moe_align_sizes",
    "moe_workspace_size", "moe_route", "moe_align", "moe_align_reroute", "moe_expert_ffn", "moe_expert_gate_up",
    "moe_expert_down", "moe_combine", "moe_forward", "moe_forward_noalloc", "moe_forward_replay",
    "moe_route_expert_choice", "NOALLOC_SCRATCH_BYTES",
    "moe_align_expert_choice", "moe_combine_expert_choice", "moe_routing_health_from_stats", "moe_routing_health",
    "MOE_ROUTE_LOGITS_IN", "MOE_ROUTE_IDS_IN", "MOE_ROUTE_NO_LOGITS_OUT",
    "MOE_OP_ALIGN",
    "MOE_OP_FORWARD", "TRACE_EVENTS", "CLOCK_SLOTS", "STATUS", "DTYPES", "ROUTING", "STATS_EXTRA", "STAT", "moe_expert_choice_sizes", "ec_capacity",
    "ec_segment",
]

MOE_F32, MOE_BF16, MOE_FP8_E4M3 = 0, 1, 2
DTYPES = {"f32": MOE_F32, "bf16": MOE_BF16, "fp8_e4m3": MOE_FP8_E4M3}
MOE_ROUTE_LOGITS_IN = 1
MOE_ROUTE_IDS_IN = 2
MOE_ROUTE_NO_LOGITS_OUT = 4
MOE_OP_ALIGN, MOE_OP_FORWARD = 1, 2
ROUTING = {"token_choice": 0, "expert_choice": 1}
STATUS = {0: "MOE_OK", 1: "MOE_ERR_NULL_POINTER", 2: "MOE_ERR_INVALID_CONFIG", 3: "MOE_ERR_UNSUPPORTED",
          4: "MOE_ERR_MISALIGNED", 5: "MOE_ERR_WORKSPACE_TOO_SMALL", 6: "MOE_ERR_HIP"}
STATS_EXTRA = 10
NOALLOC_SCRATCH_BYTES = 128 << 20  # MOE_NOALLOC_SCRATCH_BYTES
STAT = {"kept": 0, "dropped": 1, "invalid": 2, "capacity": 3, "max_load": 4, "min_load": 5, "num_padded": 6,
        "rerouted": 7, "unpicked": 8, "max_picks": 9}


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        self.name = STATUS.get(status, str(status))
        super().__init__(f"{fn} failed: {moe_status_str(status)}")


class moe_config(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32)] + [
        (n, ctypes.c_int32) for n in ("T", "H", "N", "k", "I", "B", "cap_num", "cap_den", "n_shared",
                                      "renormalize", "act_dtype", "expert_dtype", "scale_block", "reroute_depth",
                                      "routing")]


class moe_weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "w_gate", "logit_bias", "w13", "w2", "w13_scale", "w2_scale", "shared_w13", "shared_w2",
        "shared_w13_scale", "shared_w2_scale")]


class moe_trace(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "logits", "topk_ids", "topk_gates", "margin", "route_kept", "sorted_route_ids", "block_expert",
        "expert_offsets", "num_padded", "stats", "act", "y_route", "route_expert", "scores", "choice_tokens",
        "choice_slot", "choice_margin")] + [("stage_events", ctypes.POINTER(ctypes.c_void_p)),
                                             ("w13_out", ctypes.c_void_p), ("gemm_clocks", ctypes.c_void_p)]


class moe_routing_health(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "total_routes", "max_expert_load", "min_expert_load", "dropped_routes", "kept_routes", "invalid_routes",
        "capacity", "rerouted_routes", "unpicked_tokens", "reserved")] + [
        ("imbalance_ratio", ctypes.c_double), ("drop_fraction", ctypes.c_double)]


TRACE_EVENTS = 7  # router, alignment, W13, W2, shared expert, combine: 7 boundaries
CLOCK_SLOTS = 1024  # MOE_CLOCK_SLOTS


def _event_handle(e) -> Optional[int]:
    """Raw hipEvent_t of a torch.cuda.Event (created by one record on the current stream);
    None for a boundary that records no event."""
    if e is None:
        return None
    if isinstance(e, int):
        return e
    if e.cuda_event == 0:
        e.record()
    return e.cuda_event


def _trace_struct(trace: Optional[dict]):
    """moe_trace for a dict of buffers; stage_events (optional) = TRACE_EVENTS timing events
    (None entries: no event at that boundary).
    Returns (struct or None, the event array, which must outlive the call)."""
    if not trace:
        return None, None
    tr = moe_trace(**{k: _ptr(trace.get(k)) for k, _ in moe_trace._fields_ if k != "stage_events"})
    evs = trace.get("stage_events")
    arr = None
    if evs is not None:
        if len(evs) != TRACE_EVENTS:
            raise ValueError(f"stage_events: {TRACE_EVENTS} events expected, got {len(evs)}")
        arr = (ctypes.c_void_p * TRACE_EVENTS)(*[_event_handle(e) for e in evs])
        tr.stage_events = ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p))
    return tr, arr


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it is not built (there is no fallback path)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m top_routing_expert_router_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, U32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint32, ctypes.c_size_t
        cfgp = ctypes.POINTER(moe_config)
        sig = {
            "moe_abi_version": ([], I32),
            "moe_status_str": ([I32], ctypes.c_char_p),
            "moe_validate_config": ([cfgp], I32),
            "moe_align_sizes": ([cfgp, ctypes.POINTER(I32), ctypes.POINTER(I32)], I32),
            "moe_workspace_size": ([cfgp, I32, ctypes.POINTER(SZ)], I32),
            "moe_route": ([cfgp, P, P, P, P, P, P, P, U32, P], I32),
            "moe_align": ([cfgp, P, P, P, P, P, P, P, P, SZ, P], I32),
            "moe_align_reroute": ([cfgp, P, P, P, P, P, P, P, P, P, P, SZ, P], I32),
            "moe_expert_ffn": ([cfgp, P, P, P, P, P, P, P, P, P, P, P], I32),
            "moe_expert_gate_up": ([cfgp, P, P, P, P, P, P, P, P], I32),
            "moe_expert_down": ([cfgp, P, P, P, P, P, P, P], I32),
            "moe_combine": ([cfgp, P, P, P, P, P, P, P], I32),
            "moe_forward": ([cfgp, ctypes.POINTER(moe_weights), P, P, P, ctypes.POINTER(moe_trace), P, SZ, P], I32),
            "moe_forward_replay": ([cfgp, ctypes.POINTER(moe_weights), P, P, P, P, ctypes.POINTER(moe_trace), P, SZ,
                                    P], I32),
            "moe_forward_noalloc": ([cfgp, ctypes.POINTER(moe_weights), P, P, P, ctypes.POINTER(moe_trace), P], I32),
            "moe_expert_choice_sizes": ([cfgp, ctypes.POINTER(I32), ctypes.POINTER(I32)], I32),
            "moe_route_expert_choice": ([cfgp, P, P, P, P, P, P, P, P, U32, P], I32),
            "moe_align_expert_choice": ([cfgp, P, P, P, P, P, P, P, P], I32),
            "moe_combine_expert_choice": ([cfgp, P, P, P, P, P, P, P], I32),
            "moe_routing_health_from_stats": ([cfgp, P, ctypes.POINTER(moe_routing_health)], I32),
        }
        for name, (args, res) in sig.items():
            f = getattr(L, name)
            f.argtypes, f.restype = args, res
        _lib = L
    return _lib


def _ptr(x) -> Optional[int]:
    """Device address of a tensor argument (None for NULL; an int is taken as an address).
    Every tensor the C ABI reads or writes lives in device memory: a host tensor is refused
    here, before any call (a kernel given a host address faults the GPU)."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if not getattr(x, "is_cuda", False):
        raise ValueError(f"a device tensor is required, got one on {getattr(x, 'device', type(x))}")
    return x.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        if torch.cuda.is_available():
            return torch.cuda.current_stream().cuda_stream
        return None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(fn: str, st: int) -> None:
    if st != 0:
        raise MoeError(fn, st)


def make_config(T: int, H: int, N: int, k: int, I: int, B: int, *, cap_num: int = 0, cap_den: int = 0,
                n_shared: int = 0, renormalize: int = 1, act_dtype: str = "bf16", expert_dtype: str = "bf16",
                scale_block: int = 0, reroute_depth: int = 0, routing: str = "token_choice") -> moe_config:
    return moe_config(ctypes.sizeof(moe_config), T, H, N, k, I, B, cap_num, cap_den, n_shared, renormalize,
                      DTYPES[act_dtype], DTYPES[expert_dtype], scale_block, reroute_depth, ROUTING[routing])


def moe_expert_choice_sizes(cfg: moe_config):
    """Expert choice: (C tokens per expert, padded rows per expert segment)."""
    c, seg = ctypes.c_int32(), ctypes.c_int32()
    _check("moe_expert_choice_sizes",
           lib().moe_expert_choice_sizes(ctypes.byref(cfg), ctypes.byref(c), ctypes.byref(seg)))
    return c.value, seg.value


def ec_capacity(cfg: moe_config) -> int:
    return moe_expert_choice_sizes(cfg)[0]


def ec_segment(cfg: moe_config) -> int:
    return moe_expert_choice_sizes(cfg)[1]


def moe_abi_version() -> int:
    return lib().moe_abi_version()


def moe_status_str(status: int) -> str:
    return lib().moe_status_str(status).decode()


def moe_validate_config(cfg: moe_config) -> None:
    _check("moe_validate_config", lib().moe_validate_config(ctypes.byref(cfg)))


def moe_align_sizes(cfg: moe_config):
    p, n = ctypes.c_int32(), ctypes.c_int32()
    _check("moe_align_sizes", lib().moe_align_sizes(ctypes.byref(cfg), ctypes.byref(p), ctypes.byref(n)))
    return p.value, n.value


def moe_workspace_size(cfg: moe_config, op: int) -> int:
    b = ctypes.c_size_t()
    _check("moe_workspace_size", lib().moe_workspace_size(ctypes.byref(cfg), op, ctypes.byref(b)))
    return b.value


def moe_route(cfg, h, w_gate, logit_bias, logits, topk_ids, topk_gates, margin=None, flags: int = 0, stream=None):
    _check("moe_route", lib().moe_route(ctypes.byref(cfg), _ptr(h), _ptr(w_gate), _ptr(logit_bias), _ptr(logits),
                                        _ptr(topk_ids), _ptr(topk_gates), _ptr(margin), flags, _stream(stream)))


def moe_align(cfg, topk_ids, route_kept, sorted_route_ids, block_expert, expert_offsets, num_padded, stats, ws,
              ws_bytes: Optional[int] = None, stream=None):
    nb = ws_bytes if ws_bytes is not None else (ws.numel() * ws.element_size() if ws is not None else 0)
    _check("moe_align", lib().moe_align(ctypes.byref(cfg), _ptr(topk_ids), _ptr(route_kept), _ptr(sorted_route_ids),
                                        _ptr(block_expert), _ptr(expert_offsets), _ptr(num_padded), _ptr(stats),
                                        _ptr(ws), nb, _stream(stream)))


def moe_expert_ffn(cfg, h, sorted_route_ids, expert_offsets, w13, w2, w13_scale, w2_scale, act, w13_out, y_out,
                   stream=None):
    _check("moe_expert_ffn", lib().moe_expert_ffn(ctypes.byref(cfg), _ptr(h), _ptr(sorted_route_ids),
                                                  _ptr(expert_offsets), _ptr(w13), _ptr(w2), _ptr(w13_scale),
                                                  _ptr(w2_scale), _ptr(act), _ptr(w13_out), _ptr(y_out),
                                                  _stream(stream)))


def moe_expert_gate_up(cfg, h, sorted_route_ids, expert_offsets, w13, w13_scale, act, w13_out=None, stream=None):
    _check("moe_expert_gate_up", lib().moe_expert_gate_up(ctypes.byref(cfg), _ptr(h), _ptr(sorted_route_ids),
                                                          _ptr(expert_offsets), _ptr(w13), _ptr(w13_scale),
                                                          _ptr(act), _ptr(w13_out), _stream(stream)))


def moe_expert_down(cfg, act, sorted_route_ids, expert_offsets, w2, w2_scale, y_out, stream=None):
    _check("moe_expert_down", lib().moe_expert_down(ctypes.byref(cfg), _ptr(act), _ptr(sorted_route_ids),
                                                    _ptr(expert_offsets), _ptr(w2), _ptr(w2_scale), _ptr(y_out),
                                                    _stream(stream)))


def moe_combine(cfg, y_route, topk_gates, route_kept, shared_out, residual, out, stream=None):
    _check("moe_combine", lib().moe_combine(ctypes.byref(cfg), _ptr(y_route), _ptr(topk_gates), _ptr(route_kept),
                                            _ptr(shared_out), _ptr(residual), _ptr(out), _stream(stream)))


def moe_forward(cfg, weights: dict, h, residual, out, trace: Optional[dict], ws, ws_bytes: Optional[int] = None,
                stream=None):
    """weights: dict with the moe_weights member names (tensors or None); trace likewise."""
    w = moe_weights(**{k: _ptr(weights.get(k)) for k, _ in moe_weights._fields_})
    tr, _events = _trace_struct(trace)
    nb = ws_bytes if ws_bytes is not None else (ws.numel() * ws.element_size() if ws is not None else 0)
    _check("moe_forward", lib().moe_forward(ctypes.byref(cfg), ctypes.byref(w), _ptr(h), _ptr(residual), _ptr(out),
                                            ctypes.byref(tr) if tr is not None else None, _ptr(ws), nb,
                                            _stream(stream)))


def moe_forward_noalloc(cfg, weights: dict, h, residual, out, trace: Optional[dict] = None, stream=None):
    """moe_forward with its intermediates in the library's static per-GPU scratch (no workspace)."""
    w = moe_weights(**{k: _ptr(weights.get(k)) for k, _ in moe_weights._fields_})
    tr, _events = _trace_struct(trace)
    _check("moe_forward_noalloc",
           lib().moe_forward_noalloc(ctypes.byref(cfg), ctypes.byref(w), _ptr(h), _ptr(residual), _ptr(out),
                                     ctypes.byref(tr) if tr is not None else None, _stream(stream)))


def moe_forward_replay(cfg, weights: dict, h, residual, replay_ids, out, trace: Optional[dict], ws,
                       ws_bytes: Optional[int] = None, stream=None):
    """moe_forward with recorded expert ids ([T, k] int32) instead of this run's top-k."""
    w = moe_weights(**{k: _ptr(weights.get(k)) for k, _ in moe_weights._fields_})
    tr, _events = _trace_struct(trace)
    nb = ws_bytes if ws_bytes is not None else (ws.numel() * ws.element_size() if ws is not None else 0)
    _check("moe_forward_replay",
           lib().moe_forward_replay(ctypes.byref(cfg), ctypes.byref(w), _ptr(h), _ptr(residual), _ptr(replay_ids),
                                    _ptr(out), ctypes.byref(tr) if tr is not None else None, _ptr(ws), nb,
                                    _stream(stream)))


def moe_align_reroute(cfg, topk_ids, logits, route_expert, route_kept, sorted_route_ids, block_expert, expert_offsets,
                      num_padded, stats, ws, ws_bytes: Optional[int] = None, stream=None):
    """Capacity with the config's overflow policy (reroute_depth) and the alignment of the routes as they run."""
    nb = ws_bytes if ws_bytes is not None else ws.numel() * ws.element_size()
    _check("moe_align_reroute",
           lib().moe_align_reroute(ctypes.byref(cfg), _ptr(topk_ids), _ptr(logits), _ptr(route_expert),
                                   _ptr(route_kept), _ptr(sorted_route_ids), _ptr(block_expert), _ptr(expert_offsets),
                                   _ptr(num_padded), _ptr(stats), _ptr(ws), nb, _stream(stream)))


def moe_route_expert_choice(cfg, h, w_gate, logit_bias, logits, scores, choice_tokens, choice_slot,
                            choice_margin=None, flags: int = 0, stream=None):
    """Expert choice: scores [T, N] and each expert's picks (tokens [N, C], slot [T, N], margin [N])."""
    _check("moe_route_expert_choice",
           lib().moe_route_expert_choice(ctypes.byref(cfg), _ptr(h), _ptr(w_gate), _ptr(logit_bias), _ptr(logits),
                                         _ptr(scores), _ptr(choice_tokens), _ptr(choice_slot), _ptr(choice_margin),
                                         flags, _stream(stream)))


def moe_align_expert_choice(cfg, choice_tokens, choice_slot, sorted_route_ids, block_expert, expert_offsets,
                            num_padded, stats=None, stream=None):
    """Expert choice: the picks as padded rows (token ids, sentinel T) and the routing stats."""
    _check("moe_align_expert_choice",
           lib().moe_align_expert_choice(ctypes.byref(cfg), _ptr(choice_tokens), _ptr(choice_slot),
                                         _ptr(sorted_route_ids), _ptr(block_expert), _ptr(expert_offsets),
                                         _ptr(num_padded), _ptr(stats), _stream(stream)))


def moe_routing_health_from_stats(cfg, stats) -> dict:
    """Routing-health numbers of one pass from a stats array (host copy, [N + STATS_EXTRA] int32)."""
    import numpy as np
    a = np.ascontiguousarray(np.asarray(stats, dtype=np.int32))
    if a.size != cfg.N + STATS_EXTRA:
        raise ValueError(f"stats: {cfg.N + STATS_EXTRA} int32 expected, got {a.size}")
    r = moe_routing_health()
    _check("moe_routing_health_from_stats",
           lib().moe_routing_health_from_stats(ctypes.byref(cfg), a.ctypes.data, ctypes.byref(r)))
    return {k: getattr(r, k) for k, _ in moe_routing_health._fields_ if k != "reserved"}


def moe_combine_expert_choice(cfg, y_rows, scores, choice_slot, shared_out, residual, out, stream=None):
    """Expert choice: out = residual + shared + score-weighted sum of each token's picks."""
    _check("moe_combine_expert_choice",
           lib().moe_combine_expert_choice(ctypes.byref(cfg), _ptr(y_rows), _ptr(scores), _ptr(choice_slot),
                                           _ptr(shared_out), _ptr(residual), _ptr(out), _stream(stream)))
