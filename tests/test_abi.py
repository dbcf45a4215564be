"""C-ABI tests that need no GPU: the library loads, exports every declared entry
point, and rejects bad arguments on the host before any HIP call.

Every call here is built to fail validation (NULL or misaligned pointers, bad
configs), so nothing is ever enqueued on a device.
"""
import ctypes
import os
import re

import pytest

import top_routing_expert_router_amd as M
import workloads as W
from tests.harness import config

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions(header="moe.h"):
    src = open(os.path.join(ROOT, "include", header)).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_0-9]+)\s*\(", src)))


def test_library_exports_every_declared_function():
    names = _declared_functions()
    assert len(names) >= 12
    L = M.lib()
    for n in names:
        assert hasattr(L, n), n
        assert ctypes.cast(getattr(L, n), ctypes.c_void_p).value


def test_ceiling_library_exports_and_rejects_bad_arguments():
    from top_routing_expert_router_amd.build import CEILING_LIB_PATH
    L = ctypes.CDLL(CEILING_LIB_PATH)
    names = _declared_functions("moe_ceiling.h")
    assert names == ["moe_ceiling_clock_rates", "moe_ceiling_copy", "moe_ceiling_mfma_bf16", "moe_ceiling_read"]
    for n in names:
        assert ctypes.cast(getattr(L, n), ctypes.c_void_p).value
    P, SZ, I32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32
    L.moe_ceiling_copy.argtypes, L.moe_ceiling_copy.restype = [P, P, SZ, P], I32
    L.moe_ceiling_read.argtypes, L.moe_ceiling_read.restype = [P, SZ, P, P], I32
    L.moe_ceiling_mfma_bf16.argtypes, L.moe_ceiling_mfma_bf16.restype = [I32, I32, P, P], I32
    # every call below fails its host-side argument check; nothing is launched
    assert L.moe_ceiling_copy(None, 4096, 64, None) == 1
    assert L.moe_ceiling_copy(4096, 8192, 24, None) == 1
    assert L.moe_ceiling_copy(4100, 8192, 64, None) == 1
    assert L.moe_ceiling_read(4096, 0, 4096, None) == 1
    assert L.moe_ceiling_mfma_bf16(10, 3, 4096, None) == 1
    assert L.moe_ceiling_mfma_bf16(0, 1, 4096, None) == 1
    L.moe_ceiling_clock_rates.argtypes, L.moe_ceiling_clock_rates.restype = [P, P], I32
    assert L.moe_ceiling_clock_rates(None, None) == 1


def test_abi_version_and_status_strings():
    assert M.moe_abi_version() == 5
    for code, name in M.STATUS.items():
        assert M.moe_status_str(code).startswith(name)
    assert "unknown" in M.moe_status_str(99)


@pytest.mark.parametrize("w", list(W.ALL.values()), ids=list(W.ALL))
def test_workload_configs_are_valid(w):
    cfg = config(w)
    M.moe_validate_config(cfg)
    p_max, n_blocks = M.moe_align_sizes(cfg)
    act = 4 if w.act_dtype == W.F32 else 2
    fwd = M.moe_workspace_size(cfg, M.MOE_OP_FORWARD)
    if w.routing == "expert_choice":
        C, seg = M.moe_expert_choice_sizes(cfg)
        assert C == min(w.T * w.k * (w.cap_num or 1) // (w.N * (w.cap_den or 1)), w.T)
        assert seg == -(-C // w.B) * w.B and p_max == w.N * seg and n_blocks == p_max // w.B
        assert M.moe_workspace_size(cfg, M.MOE_OP_ALIGN) == 0
        assert fwd >= p_max * (w.I + w.H) * act + 3 * w.T * w.N * 4
        return
    assert p_max == w.T * w.k + w.N * (w.B - 1)
    assert n_blocks == -(-p_max // w.B)
    assert M.moe_workspace_size(cfg, M.MOE_OP_ALIGN) > 0
    assert fwd >= p_max * w.I * act + w.T * w.k * w.H * act


BAD = [
    dict(T=0), dict(T=65537), dict(H=100), dict(H=0), dict(I=64), dict(N=0), dict(N=257), dict(k=0),
    dict(k=9, N=16), dict(k=3, N=2), dict(B=12), dict(B=256), dict(cap_num=5, cap_den=0),
    dict(cap_num=-1, cap_den=4), dict(n_shared=2), dict(renormalize=2), dict(T=65536, H=32768),
    dict(I=32768, H=32768), dict(reroute_depth=-1), dict(reroute_depth=7, N=8, k=2),
    dict(routing=2), dict(routing=-1), dict(routing=1, reroute_depth=1, cap_num=1, cap_den=1),
]


@pytest.mark.parametrize("bad", BAD, ids=[str(b) for b in BAD])
def test_invalid_configs_rejected(bad):
    routing = bad.pop("routing", 0)
    cfg = config(W.MIXTRAL_BF16, **bad)
    cfg.routing = routing
    with pytest.raises(M.MoeError) as ei:
        M.moe_validate_config(cfg)
    assert ei.value.name == "MOE_ERR_INVALID_CONFIG"


def test_unsupported_dtype_combinations():
    for act, exp, sb in (("f32", "bf16", 0), ("bf16", "f32", 0), ("f32", "fp8_e4m3", 128), ("bf16", "fp8_e4m3", 64)):
        cfg = M.make_config(64, 128, 8, 2, 256, 8, act_dtype=act, expert_dtype=exp, scale_block=sb)
        with pytest.raises(M.MoeError) as ei:
            M.moe_validate_config(cfg)
        assert ei.value.name == "MOE_ERR_UNSUPPORTED"
    cfg = config(W.MIXTRAL_BF16)
    cfg.struct_size = 8
    with pytest.raises(M.MoeError):
        M.moe_validate_config(cfg)


def _expect(name, fn, *args, **kw):
    with pytest.raises(M.MoeError) as ei:
        fn(*args, **kw)
    assert ei.value.name == name, ei.value


def test_host_validation_of_pointers_and_workspace():
    cfg = config(W.MIXTRAL_BF16)
    A, ODD = 4096, 4098  # stand-in addresses: never dereferenced, every call below fails validation
    s = 0
    # route
    _expect("MOE_ERR_NULL_POINTER", M.moe_route, cfg, A, A, None, None, A, A, None, 0, s)
    _expect("MOE_ERR_NULL_POINTER", M.moe_route, cfg, None, A, None, A, A, A, None, 0, s)
    _expect("MOE_ERR_MISALIGNED", M.moe_route, cfg, ODD, A, None, A, A, A, None, 0, s)
    _expect("MOE_ERR_MISALIGNED", M.moe_route, cfg, A, A, None, A + 1, A, A, None, M.MOE_ROUTE_LOGITS_IN, s)
    _expect("MOE_ERR_UNSUPPORTED", M.moe_route, cfg, A, A, None, A, A, A, None, 0x10, s)
    # no logits out: not with given logits, not on the fp32 path (it stages them in `logits`)
    _expect("MOE_ERR_UNSUPPORTED", M.moe_route, cfg, A, A, None, A, A, A, None,
            M.MOE_ROUTE_NO_LOGITS_OUT | M.MOE_ROUTE_LOGITS_IN, s)
    _expect("MOE_ERR_UNSUPPORTED", M.moe_route, config(W.TOY_FP32), A, A, None, None, A, A, None,
            M.MOE_ROUTE_NO_LOGITS_OUT, s)
    _expect("MOE_ERR_NULL_POINTER", M.moe_route, cfg, A, A, None, None, None, A, None, M.MOE_ROUTE_NO_LOGITS_OUT, s)
    # align
    _expect("MOE_ERR_NULL_POINTER", M.moe_align, cfg, A, A, A, A, A, None, None, A, 1 << 20, s)
    _expect("MOE_ERR_MISALIGNED", M.moe_align, cfg, A + 2, A, A, A, A, A, None, A, 1 << 20, s)
    _expect("MOE_ERR_WORKSPACE_TOO_SMALL", M.moe_align, cfg, A, A, A, A, A, A, None, A, 4, s)
    # expert ffn
    _expect("MOE_ERR_NULL_POINTER", M.moe_expert_ffn, cfg, A, A, None, A, A, None, None, A, None, A, s)
    _expect("MOE_ERR_NULL_POINTER", M.moe_expert_ffn, cfg, A, None, None, None, A, None, None, A, None, A, s)
    _expect("MOE_ERR_MISALIGNED", M.moe_expert_ffn, cfg, A, None, None, A, A, None, None, A + 8, None, A, s)
    _expect("MOE_ERR_MISALIGNED", M.moe_expert_ffn, cfg, A, None, None, A, A, None, None, A, A + 8, A, s)
    _expect("MOE_ERR_MISALIGNED", M.moe_expert_gate_up, cfg, A, None, None, A, None, A, A + 2, s)
    _expect("MOE_ERR_NULL_POINTER", M.moe_expert_gate_up, cfg, A, A, None, A, None, A, A, s)
    cfg8 = config(W.DEEPSEEKV3_FP8)
    _expect("MOE_ERR_NULL_POINTER", M.moe_expert_ffn, cfg8, A, None, None, A, A, None, None, A, None, A, s)
    # combine
    _expect("MOE_ERR_NULL_POINTER", M.moe_combine, cfg, A, A, None, None, None, A, s)
    _expect("MOE_ERR_MISALIGNED", M.moe_combine, cfg, A, A, A, None, ODD, A, s)
    # forward
    _expect("MOE_ERR_NULL_POINTER", M.moe_forward, cfg, {"w_gate": A, "w13": A}, A, None, A, None, A, 1 << 40, s)
    full = {"w_gate": A, "w13": A, "w2": A}
    _expect("MOE_ERR_WORKSPACE_TOO_SMALL", M.moe_forward, cfg, full, A, None, A, None, A, 1024, s)
    _expect("MOE_ERR_MISALIGNED", M.moe_forward, cfg, full, A, None, A, None, A + 16, 1 << 40, s)
    _expect("MOE_ERR_NULL_POINTER", M.moe_forward, cfg8, full, A, None, A, None, A, 1 << 40, s)
    bad = config(W.MIXTRAL_BF16, k=0)
    _expect("MOE_ERR_INVALID_CONFIG", M.moe_forward, bad, full, A, None, A, None, A, 1 << 40, s)
    # forward replay: the recorded ids are required and 4-byte aligned; the rest as moe_forward
    _expect("MOE_ERR_NULL_POINTER", M.moe_forward_replay, cfg, full, A, None, None, A, None, A, 1 << 40, s)
    _expect("MOE_ERR_MISALIGNED", M.moe_forward_replay, cfg, full, A, None, A + 2, A, None, A, 1 << 40, s)
    _expect("MOE_ERR_WORKSPACE_TOO_SMALL", M.moe_forward_replay, cfg, full, A, None, A, A, None, A, 1024, s)
    _expect("MOE_ERR_INVALID_CONFIG", M.moe_forward_replay, bad, full, A, None, A, A, None, A, 1 << 40, s)
    # reroute alignment: logits and route_expert are required
    cs = config(W.SWITCH_BF16, reroute_depth=2)
    _expect("MOE_ERR_NULL_POINTER", M.moe_align_reroute, cs, A, None, A, A, A, A, A, A, None, A, 1 << 20, s)
    _expect("MOE_ERR_NULL_POINTER", M.moe_align_reroute, cs, A, A, None, A, A, A, A, A, None, A, 1 << 20, s)
    _expect("MOE_ERR_MISALIGNED", M.moe_align_reroute, cs, A, A + 2, A, A, A, A, A, A, None, A, 1 << 20, s)
    _expect("MOE_ERR_WORKSPACE_TOO_SMALL", M.moe_align_reroute, cs, A, A, A, A, A, A, A, A, None, A, 64, s)
    # route with recorded ids: the flag is known; unknown bits are not
    _expect("MOE_ERR_NULL_POINTER", M.moe_route, cfg, A, A, None, A, None, A, None, M.MOE_ROUTE_IDS_IN, s)
    _expect("MOE_ERR_UNSUPPORTED", M.moe_route, cfg, A, A, None, A, A, A, None, 0x8 | M.MOE_ROUTE_IDS_IN, s)


def test_workspace_op_codes():
    cfg = config(W.TOY_FP32)
    _expect("MOE_ERR_INVALID_CONFIG", M.moe_workspace_size, cfg, 7)


def test_routing_mode_mismatch_is_unsupported():
    tc, ec = config(W.MIXTRAL_BF16), config(W.MIXTRAL_EC_BF16)
    A = 4096  # stand-in address: every call below fails validation, nothing is enqueued
    s = 0
    full = {"w_gate": A, "w13": A, "w2": A}
    # token-choice entry points refuse an expert-choice config
    _expect("MOE_ERR_UNSUPPORTED", M.moe_route, ec, A, A, None, A, A, A, None, 0, s)
    _expect("MOE_ERR_UNSUPPORTED", M.moe_align, ec, A, A, A, A, A, A, None, A, 1 << 20, s)
    _expect("MOE_ERR_UNSUPPORTED", M.moe_align_reroute, ec, A, A, A, A, A, A, A, A, None, A, 1 << 20, s)
    _expect("MOE_ERR_UNSUPPORTED", M.moe_combine, ec, A, A, A, None, None, A, s)
    _expect("MOE_ERR_UNSUPPORTED", M.moe_forward_replay, ec, full, A, None, A, A, None, A, 1 << 40, s)
    # and the expert-choice ones a token-choice config
    _expect("MOE_ERR_UNSUPPORTED", M.moe_expert_choice_sizes, tc)
    _expect("MOE_ERR_UNSUPPORTED", M.moe_route_expert_choice, tc, A, A, None, A, A, A, A, None, 0, s)
    _expect("MOE_ERR_UNSUPPORTED", M.moe_align_expert_choice, tc, A, A, A, A, A, A, None, s)
    _expect("MOE_ERR_UNSUPPORTED", M.moe_combine_expert_choice, tc, A, A, A, None, None, A, s)


def test_expert_choice_host_validation():
    ec = config(W.MIXTRAL_EC_BF16)
    A, s = 4096, 0
    _expect("MOE_ERR_NULL_POINTER", M.moe_route_expert_choice, ec, A, A, None, None, A, A, A, None, 0, s)
    _expect("MOE_ERR_NULL_POINTER", M.moe_route_expert_choice, ec, A, A, None, A, None, A, A, None, 0, s)
    _expect("MOE_ERR_NULL_POINTER", M.moe_route_expert_choice, ec, A, A, None, A, A, None, A, None, 0, s)
    _expect("MOE_ERR_NULL_POINTER", M.moe_route_expert_choice, ec, None, A, None, A, A, A, A, None, 0, s)
    _expect("MOE_ERR_MISALIGNED", M.moe_route_expert_choice, ec, A, A, None, A, A + 2, A, A, None, 0, s)
    _expect("MOE_ERR_MISALIGNED", M.moe_route_expert_choice, ec, A + 8, A, None, A, A, A, A, None, 0, s)
    _expect("MOE_ERR_UNSUPPORTED", M.moe_route_expert_choice, ec, A, A, None, A, A, A, A, None,
            M.MOE_ROUTE_IDS_IN, s)
    _expect("MOE_ERR_NULL_POINTER", M.moe_align_expert_choice, ec, None, A, A, A, A, A, None, s)
    _expect("MOE_ERR_NULL_POINTER", M.moe_align_expert_choice, ec, A, None, A, A, A, A, A, s)
    _expect("MOE_ERR_MISALIGNED", M.moe_align_expert_choice, ec, A, A, A + 1, A, A, A, None, s)
    _expect("MOE_ERR_NULL_POINTER", M.moe_combine_expert_choice, ec, A, A, None, None, None, A, s)
    _expect("MOE_ERR_MISALIGNED", M.moe_combine_expert_choice, ec, A + 4, A, A, None, None, A, s)
    full = {"w_gate": A, "w13": A, "w2": A}
    _expect("MOE_ERR_WORKSPACE_TOO_SMALL", M.moe_forward, ec, full, A, None, A, None, A, 1024, s)
    assert M.moe_expert_choice_sizes(ec) == (1024, 1024)
    assert M.moe_expert_choice_sizes(config(W.MIXTRAL_EC_BF16, T=5, cap_num=1, cap_den=1)) == (1, 64)
    assert M.moe_expert_choice_sizes(config(W.MIXTRAL_EC_BF16, T=3, k=1)) == (0, 0)


def _header_fields(struct: str):
    """Member names of a struct in include/moe.h, in declaration order."""
    import os
    import re
    text = open(os.path.join(os.path.dirname(__file__), "..", "include", "moe.h")).read()
    body = re.search(r"typedef struct %s \{(.*?)\} %s;" % (struct, struct), text, re.S).group(1)
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    return [re.search(r"(\w+)\s*(\[[^\]]*\])?\s*$", d.strip()).group(1) for d in body.split(";") if d.strip()]


def test_binding_structs_match_the_header():
    # the ctypes mirrors must list the C members in the same order (all pointer-sized here)
    assert [n for n, _ in M.moe_trace._fields_] == _header_fields("moe_trace")
    assert [n for n, _ in M.moe_weights._fields_] == _header_fields("moe_weights")
    assert [n for n, _ in M.moe_routing_health._fields_] == _header_fields("moe_routing_health")
    assert M.TRACE_EVENTS == 7


def _stats_array(N, load, kept, dropped, invalid, cap, rerouted=0, unpicked=0):
    """A stats array laid out as the alignment writes it: per-expert load, then the counters."""
    import numpy as np
    st = np.zeros(N + M.STATS_EXTRA, np.int32)
    st[:N] = load
    x = N
    st[x + M.STAT["kept"]], st[x + M.STAT["dropped"]], st[x + M.STAT["invalid"]] = kept, dropped, invalid
    st[x + M.STAT["capacity"]] = cap
    st[x + M.STAT["max_load"]], st[x + M.STAT["min_load"]] = max(load), min(load)
    st[x + M.STAT["rerouted"]], st[x + M.STAT["unpicked"]] = rerouted, unpicked
    return st


def test_routing_health_from_stats_matches_the_oracle_probe():
    # host-only helper: the numbers of the routing-stats probe from a stats array, against
    # the oracle's routing_stats on the same routes (drop policy, with and without capacity)
    import numpy as np
    from oracle import moe_oracle as O
    rng = np.random.default_rng(4)
    for T, N, k, cf in ((64, 8, 2, None), (300, 16, 1, (5, 4)), (33, 6, 3, (1, 2)), (5, 4, 2, (1, 8))):
        ids = rng.integers(-1, N + 1, size=(T, k)) if T == 33 else (rng.zipf(1.6, size=(T, k)) - 1) % N
        cap = O.capacity(T, k, N, *(cf or (0, 0)))
        kept = O.capacity_keep(ids, N, cap)
        ref = O.routing_stats(ids, kept, N, cap)
        cfg = config(W.MIXTRAL_BF16, T=T, N=N, k=k, cap_num=cf[0] if cf else 0, cap_den=cf[1] if cf else 0)
        st = _stats_array(N, ref["load"], ref["kept_routes"], ref["dropped_tokens"], ref["invalid_routes"],
                          ref["capacity"])
        got = M.moe_routing_health_from_stats(cfg, st)
        assert got["max_expert_load"] == ref["max_expert_load"] and got["min_expert_load"] == ref["min_expert_load"]
        assert got["dropped_routes"] == ref["dropped_tokens"] and got["kept_routes"] == ref["kept_routes"]
        assert got["invalid_routes"] == ref["invalid_routes"] and got["capacity"] == ref["capacity"]
        assert got["total_routes"] == int(ref["load"].sum())
        assert got["imbalance_ratio"] == pytest.approx(ref["imbalance_ratio"], rel=1e-15, abs=0)
        assert got["drop_fraction"] == pytest.approx(ref["drop_fraction"], rel=1e-15, abs=0)
    # no valid route: both ratios are 0
    cfg = config(W.MIXTRAL_BF16, T=2, N=4, k=1)
    z = M.moe_routing_health_from_stats(cfg, _stats_array(4, [0, 0, 0, 0], 0, 0, 2, -1))
    assert z["imbalance_ratio"] == 0.0 and z["drop_fraction"] == 0.0 and z["invalid_routes"] == 2


def test_routing_health_rejects_bad_arguments():
    import numpy as np
    cfg = config(W.MIXTRAL_BF16)
    r = M.moe_routing_health()
    L = M.lib()
    st = np.zeros(cfg.N + M.STATS_EXTRA, np.int32)
    assert L.moe_routing_health_from_stats(ctypes.byref(cfg), None, ctypes.byref(r)) == 1
    assert L.moe_routing_health_from_stats(ctypes.byref(cfg), st.ctypes.data, None) == 1
    st[0] = -3  # a negative load: no alignment writes that
    assert L.moe_routing_health_from_stats(ctypes.byref(cfg), st.ctypes.data, ctypes.byref(r)) == 2
    bad = config(W.MIXTRAL_BF16, k=0)
    assert L.moe_routing_health_from_stats(ctypes.byref(bad), np.zeros(18, np.int32).ctypes.data, ctypes.byref(r)) == 2


def test_stage_events_argument_checked_by_the_binding():
    with pytest.raises(ValueError):
        M._trace_struct({"stage_events": [0, 0, 0]})
    tr, arr = M._trace_struct({"stage_events": [0] * M.TRACE_EVENTS})
    assert arr is not None and len(arr) == M.TRACE_EVENTS
