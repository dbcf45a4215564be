#!/usr/bin/env python3
"""Throughput of the MoE layer forward pass on one MI355X.

A step is one moe_forward call (router projection, top-k + gates, capacity +
alignment, grouped W13+SwiGLU and W2 expert GEMMs, combine) over one batch of
seeded synthetic inputs already resident in HBM.  Default workload: the
Mixtral-shaped layer (T=4096, H=4096, 8 experts, top-2, SwiGLU I=14336, B=64,
bf16).  Prints ONE JSON line on stdout; progress goes to stderr.

The expert GEMMs are timed inside the timed steps themselves, by HIP events the
forward records on its stream around them (its trace's stage events, at those
boundaries only); the dominant one (the W13+SwiGLU grouped GEMM) is reported
against the bf16 MFMA peak.  Every other stage is timed in forwards carrying all
the stage events and on its own (cold), and the CPU oracle on a bounded token
sample.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = "routed tokens/sec per MoE layer fwd (1 GPU) + % MFMA/HBM roofline"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class TimingEvent:
    """A HIP event for timing only, created with hipEventDisableSystemFence: recording it
    does no system-scope cache write-back and invalidation (which a default event does, and
    which costs the kernels around it several microseconds).  The library records it where a
    trace's stage_events put it; elapsed() reads the time between two recorded events."""
    _hip = None
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes
        if TimingEvent._hip is None:
            TimingEvent._hip = ctypes.CDLL("libamdhip64.so")
        self._ev = ctypes.c_void_p()
        err = TimingEvent._hip.hipEventCreateWithFlags(ctypes.byref(self._ev), self.DISABLE_SYSTEM_FENCE)
        if err != 0:
            raise RuntimeError(f"hipEventCreateWithFlags: error {err}")
        self.handle = self._ev.value

    def elapsed_time(self, end: "TimingEvent") -> float:
        import ctypes
        ms = ctypes.c_float()
        err = TimingEvent._hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(self.handle),
                                                   ctypes.c_void_p(end.handle))
        if err != 0:
            raise RuntimeError(f"hipEventElapsedTime: error {err}")
        return ms.value

    def __del__(self):
        if TimingEvent._hip is not None and getattr(self, "handle", None):
            import ctypes
            TimingEvent._hip.hipEventDestroy(ctypes.c_void_p(self.handle))


def _ffn_source_hash() -> str:
    """Hash of the GEMM source's code (comments and blank space removed), which the
    committed traffic counters were taken on."""
    import re
    p = os.path.join(ROOT, "top_routing_expert_router_amd", "csrc", "ffn.hip")
    src = open(p).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    src = re.sub(r"//[^\n]*", "", src)
    src = "\n".join(line.strip() for line in src.splitlines() if line.strip())
    return hashlib.sha256(src.encode()).hexdigest()[:16]


def _traffic(workload: str, launches_per_unit: float):
    """HBM bytes per launch of the W13 GEMM from committed rocprofv3 counter runs,
    if they were taken on the current kernel source; else None."""
    p = os.path.join(ROOT, "profiles", f"gate_up_gemm_{workload}_traffic.json")
    if not os.path.exists(p):
        return None
    d = json.load(open(p))
    if d.get("ffn_source_sha256_16") != _ffn_source_hash():
        return None
    return d.get("hbm_bytes_per_launch")


# rocprofv3 kernel-name fragments -> stage names used in the counter summary
_COUNTER_KERNELS = [("ffn_gemm_bf16<0", "gate_up_gemm"), ("ffn_gemm_bf16<1", "down_gemm"),
                    ("router_ring", "route_ring"), ("router_bf16", "route"), ("topk_gates", "route_topk"),
                    ("align_hist", "align_hist"), ("align_scan", "align_scan"), ("align_scatter", "align_scatter"),
                    ("align_fused", "align_one_workgroup"), ("ec_select", "expert_choice_select"),
                    ("ec_align_init", "align_ec_init"), ("ec_align_rows", "align_ec_rows"), ("combine_ec_rows", "combine_expert_choice"),
                    ("reroute_rank", "reroute_rank"), ("reroute_capacity", "reroute"),
                    ("combine_rows", "combine"), ("copy16", "ceiling_copy_1GiB"), ("read16", "ceiling_read_1GiB"),
                    ("mfma_loop<1>", "ceiling_mfma_1wave"), ("mfma_loop<2>", "ceiling_mfma_2wave")]


def summarize_counters(fetch_dir: str, write_dir: str, workload: str, out_dir: str = None) -> int:
    """Turn two rocprofv3 --pmc runs of this script (FETCH_SIZE, then WRITE_SIZE; CSV
    output) into HBM bytes per launch.  Both counters are in KiB per dispatch; each is
    scaled by bytes / counter for the 1 GiB copy kernel the same runs launch (it reads
    and writes exactly 2^30 bytes).  Writes gate_up_gemm_<workload>_traffic.json into
    out_dir (default profiles/), tagged with the hash of the GEMM source it was taken on,
    and prints a text summary."""
    import csv
    import statistics

    def per_kernel(d, counter):
        path = os.path.join(d, "run_counter_collection.csv")
        vals = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            for frag, stage in _COUNTER_KERNELS:
                if frag in r["Kernel_Name"]:
                    vals.setdefault(stage, []).append(float(r["Counter_Value"]))
        return {k: statistics.mean(v) for k, v in vals.items()}, {k: len(v) for k, v in vals.items()}

    fetch, nf = per_kernel(fetch_dir, "FETCH_SIZE")
    write, nw = per_kernel(write_dir, "WRITE_SIZE")
    copy_bytes = float(1 << 30)
    f_scale = copy_bytes / (fetch["ceiling_copy_1GiB"] * 1024)
    w_scale = copy_bytes / (write["ceiling_copy_1GiB"] * 1024)
    rows = {}
    for stage in fetch:
        if stage not in write:
            continue
        rb, wb = fetch[stage] * 1024 * f_scale, write[stage] * 1024 * w_scale
        rows[stage] = {"fetch_KiB": round(fetch[stage], 1), "write_KiB": round(write[stage], 1),
                       "read_bytes": round(rb), "write_bytes": round(wb), "hbm_bytes": round(rb + wb),
                       "dispatches": nf[stage]}
    out = {"workload": workload, "ffn_source_sha256_16": _ffn_source_hash(),
           "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4),
           "hbm_bytes_per_launch": rows["gate_up_gemm"]["hbm_bytes"], "kernels": rows}
    path = os.path.join(out_dir or os.path.join(ROOT, "profiles"), f"gate_up_gemm_{workload}_traffic.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(f"counter calibration: FETCH_SIZE x{f_scale:.4f}, WRITE_SIZE x{w_scale:.4f} "
          f"(1 GiB copy kernel: {fetch['ceiling_copy_1GiB']:.0f} / {write['ceiling_copy_1GiB']:.0f} KiB)")
    print(f"{'kernel':<20}{'FETCH KiB':>14}{'WRITE KiB':>14}{'read GB':>10}{'write GB':>10}{'HBM GB':>10}")
    for k, v in rows.items():
        print(f"{k:<20}{v['fetch_KiB']:>14,.0f}{v['write_KiB']:>14,.0f}{v['read_bytes'] / 1e9:>10.4f}"
              f"{v['write_bytes'] / 1e9:>10.4f}{v['hbm_bytes'] / 1e9:>10.4f}")
    print(f"wrote {path}")
    return 0


def summarize_trace(trace_dir: str, workload: str, warmup: int = 0, steps: int = 0) -> int:
    """Per-kernel durations from a rocprofv3 --kernel-trace run of this script (CSV
    output): calls, average, min, max and share of GPU time, layer kernels by name
    and torch's own kernels (input generation, cache-flush fills) lumped together.
    With warmup and steps (those of the traced run), also the layer's kernels over the
    timed steps alone, picked by dispatch order: the script's first calls of the layer are
    the warmup forwards, then the timed ones.  With a shared expert each forward launches
    each GEMM kernel twice (routed experts first, then the shared expert); the two are
    reported apart."""
    import csv
    import statistics

    import workloads as W

    per, order = {}, {}
    rows = list(csv.DictReader(open(os.path.join(trace_dir, "run_kernel_trace.csv"))))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    for r in rows:
        n = r["Kernel_Name"]
        name = next((st for frag, st in _COUNTER_KERNELS if frag in n), None)
        if name is None:
            name = "torch (inputs, flush fills)" if "at::native" in n else n.split("(")[0][-40:]
        us = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        per.setdefault(name, []).append(us)
    total = sum(sum(v) for v in per.values())
    print(f"# rocprofv3 kernel trace of bench.py, workload {workload}; durations in microseconds")
    print(f"{'kernel':<30}{'calls':>7}{'avg_us':>11}{'min_us':>11}{'max_us':>11}{'total_us':>12}{'pct':>8}")
    for k, v in sorted(per.items(), key=lambda kv: -sum(kv[1])):
        print(f"{k:<30}{len(v):>7}{statistics.mean(v):>11.2f}{min(v):>11.2f}{max(v):>11.2f}"
              f"{sum(v):>12.1f}{100 * sum(v) / total:>8.2f}")
    if steps > 0:
        shared = W.ALL[workload].n_shared > 0 if workload in W.ALL else False
        print(f"# the {steps} timed steps alone (launches {warmup} .. {warmup + steps - 1} of each layer kernel, "
              f"in dispatch order)")
        print(f"{'kernel':<30}{'calls':>7}{'avg_us':>11}{'min_us':>11}{'max_us':>11}")
        for k, v in per.items():
            if k.startswith("ceiling") or k.startswith("torch") or k.startswith("__"):
                continue
            gemm = k in ("gate_up_gemm", "down_gemm")
            per_fwd = 2 if gemm and shared else 1
            if len(v) < per_fwd * (warmup + steps):
                continue  # not launched by every forward (a standalone call elsewhere in the script)
            sel = v[per_fwd * warmup: per_fwd * (warmup + steps)]
            parts = [(k, sel)] if per_fwd == 1 else [(k + " (routed)", sel[0::2]), (k + " (shared)", sel[1::2])]
            for name, x in parts:
                if x:
                    print(f"{name:<30}{len(x):>7}{statistics.mean(x):>11.2f}{min(x):>11.2f}{max(x):>11.2f}")
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="mixtral_bf16")
    ap.add_argument("--cpu-sample", type=int, default=0,
                    help="tokens of the workload the CPU oracle runs (default 0: the whole batch, about 6 s of "
                         "host work on the Mixtral-shaped layer)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-stages", action="store_true", help="skip the per-stage timings")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="no GPU: summarize two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of this script")
    ap.add_argument("--summarize-trace", metavar="TRACE_DIR",
                    help="no GPU: per-kernel durations from a rocprofv3 --kernel-trace run of this script "
                         "(give that run's --steps and --warmup to also get its timed steps alone)")
    args = ap.parse_args()
    if args.summarize_trace:
        return summarize_trace(args.summarize_trace, args.workload, args.warmup, args.steps)
    if args.summarize_counters:
        return summarize_counters(*args.summarize_counters, args.workload)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(expert parallelism is a design note); run with --gpus 1.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import top_routing_expert_router_amd as M
    import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    M.lib()
    dev = "cuda"
    w = W.ALL[args.workload]
    log(f"[bench] workload {w.name}: generating inputs on the GPU")
    d = W.layer_inputs(w, device=dev)
    cfg = M.make_config(w.T, w.H, w.N, w.k, w.I, w.B, cap_num=w.cap_num, cap_den=w.cap_den, n_shared=w.n_shared,
                        renormalize=w.renormalize, act_dtype=w.act_dtype, expert_dtype=w.expert_dtype,
                        scale_block=w.scale_block, reroute_depth=w.reroute_depth, routing=w.routing)
    p_max, n_blocks = M.moe_align_sizes(cfg)
    ec = w.routing == "expert_choice"
    C = M.moe_expert_choice_sizes(cfg)[0] if ec else 0
    act_t = torch.float32 if w.act_dtype == W.F32 else torch.bfloat16
    asz = 4 if w.act_dtype == W.F32 else 2
    ws = torch.empty(M.moe_workspace_size(cfg, M.MOE_OP_FORWARD), dtype=torch.uint8, device=dev)
    out = torch.empty(w.T, w.H, dtype=act_t, device=dev)
    wts = {k: d.get(k) for k in ("w_gate", "w13", "w2", "w13_scale", "w2_scale", "shared_w13", "shared_w2",
                                 "shared_w13_scale", "shared_w2_scale")}
    wts["logit_bias"] = None if d["bias"] is None else d["bias"].to(dev)
    stream = torch.cuda.current_stream()

    def step(trace=None):
        M.moe_forward(cfg, wts, d["h"], d["residual"], out, trace, ws, stream=stream)

    # events around the expert GEMMs inside every timed step (boundaries: after the alignment,
    # after W13, after W2, and after the shared expert when there is one): the GEMM times come
    # from the timed region itself, from the launches the step time covers.  Each event is a
    # packet of its own on the stream, so no more are recorded than these times need, and they
    # are timing-only events (no system-scope fence).
    gemm_ev = [[None, None] + [TimingEvent() for _ in range(3)] + [TimingEvent() if w.n_shared else None, None]
               for _ in range(args.steps)]
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for i in range(args.steps):
        step({"stage_events": [None if e is None else e.handle for e in gemm_ev[i]]})
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    value = w.T / (ms / 1e3)
    timed_gemm_ms = [sum(ev[b].elapsed_time(ev[b + 1]) for ev in gemm_ev) / args.steps
                     for b in ((2, 3, 4) if w.n_shared else (2, 3))]
    log(f"[bench] forward: {ms:.4f} ms/step, {value:,.0f} tokens/s")
    log(f"[bench] inside the timed steps: W13 {timed_gemm_ms[0] * 1e3:,.1f} us, W2 {timed_gemm_ms[1] * 1e3:,.1f} us"
        + (f", shared expert {timed_gemm_ms[2] * 1e3:,.1f} us" if w.n_shared else ""))

    # ---- per-stage timings through the individual entry points (same buffers)
    tr = dict(logits=torch.empty(w.T, w.N, device=dev),
              sorted_route_ids=torch.empty(max(p_max, 1), dtype=torch.int32, device=dev),
              block_expert=torch.empty(max(n_blocks, 1), dtype=torch.int32, device=dev),
              expert_offsets=torch.empty(w.N + 1, dtype=torch.int32, device=dev),
              num_padded=torch.empty(1, dtype=torch.int32, device=dev),
              stats=torch.empty(w.N + M.STATS_EXTRA, dtype=torch.int32, device=dev),
              act=torch.empty(max(p_max, 1), w.I, dtype=act_t, device=dev))
    if ec:
        tr.update(scores=torch.empty(w.T, w.N, device=dev),
                  choice_tokens=torch.empty(max(w.N * C, 1), dtype=torch.int32, device=dev),
                  choice_slot=torch.empty(w.T, w.N, dtype=torch.int32, device=dev),
                  choice_margin=torch.empty(w.N, device=dev),
                  y_route=torch.empty(max(p_max, 1), w.H, dtype=act_t, device=dev))
    else:
        tr.update(topk_ids=torch.empty(w.T, w.k, dtype=torch.int32, device=dev),
                  topk_gates=torch.empty(w.T, w.k, device=dev), margin=torch.empty(w.T, device=dev),
                  route_kept=torch.empty(w.T * w.k, dtype=torch.uint8, device=dev),
                  y_route=torch.empty(w.T * w.k, w.H, dtype=act_t, device=dev))
    M.moe_forward(cfg, wts, d["h"], d["residual"], out, tr, ws, stream=stream)
    torch.cuda.synchronize()
    kept_routes = w.N * C if ec else int(tr["route_kept"].sum().item())
    aws = torch.empty(M.moe_workspace_size(cfg, M.MOE_OP_ALIGN), dtype=torch.uint8, device=dev)
    # cold runs: a read of 1 GiB (more than L2 and MALL together) before each timed launch
    # evicts what the caches hold without leaving dirty lines for the timed kernel to write back
    flush = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
    flush_sink = torch.zeros(4096, dtype=torch.float32, device=dev)
    read_1gib = ceiling_reader(flush, flush_sink, stream)

    def timed(fn, reps, do_flush):
        es = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        fn()
        for a, b in es:
            if do_flush:
                read_1gib()
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        return sum(a.elapsed_time(b) for a, b in es) / reps  # ms per launch

    def in_forward(reps):
        """Stage times inside the layer: moe_forward with the trace's stage events (the
        kernels exactly as the forward launches them, each seeing the clocks and caches it
        sees there).  ms per stage: route, align, W13, W2, shared expert, combine."""
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(M.TRACE_EVENTS)] for _ in range(reps)]
        M.moe_forward(cfg, wts, d["h"], d["residual"], out, {"stage_events": evs[0]}, ws, stream=stream)
        torch.cuda.synchronize()
        for ev in evs:
            M.moe_forward(cfg, wts, d["h"], d["residual"], out, {"stage_events": ev}, ws, stream=stream)
        torch.cuda.synchronize()
        stage = [sum(ev[i].elapsed_time(ev[i + 1]) for ev in evs) / reps for i in range(M.TRACE_EVENTS - 1)]
        whole = sum(ev[0].elapsed_time(ev[-1]) for ev in evs) / reps
        return stage, whole

    R, T, H, I, N, k = w.T * w.k, w.T, w.H, w.I, w.N, w.k
    stages = {}
    gate_up_flops = 4.0 * kept_routes * H * I
    down_flops = 2.0 * kept_routes * H * I
    fwd_stage_ms, fwd_events_ms = in_forward(max(args.steps, 5))
    ms_gate_up, ms_down = timed_gemm_ms[0], timed_gemm_ms[1]
    stages["gate_up_gemm"] = {"us": ms_gate_up * 1e3, "TFLOP/s": gate_up_flops / (ms_gate_up * 1e-3) / 1e12}
    stages["down_gemm"] = {"us": ms_down * 1e3, "TFLOP/s": down_flops / (ms_down * 1e-3) / 1e12}
    if w.n_shared:
        sh_flops = 6.0 * T * H * I * w.n_shared
        stages["shared_expert"] = {"us": timed_gemm_ms[2] * 1e3,
                                   "TFLOP/s": sh_flops / (timed_gemm_ms[2] * 1e-3) / 1e12}
    if not args.no_stages and ec:
        ec_stages(stages, w, cfg, d, wts, tr, out, ws, C, p_max, n_blocks, asz, timed, max(args.steps, 5), stream)
        for name, ms_stage in (("route_expert_choice", fwd_stage_ms[0]), ("align_expert_choice", fwd_stage_ms[1]),
                               ("combine", fwd_stage_ms[5])):
            stages[name]["in_forward_us"] = ms_stage * 1e3
        for kname, v in stages.items():
            log(f"[bench] stage {kname}: " + ", ".join(f"{a} {b:,.2f}" for a, b in v.items()))
    elif not args.no_stages:
        route_bytes = T * H * asz + N * H * asz + T * N * 4 + R * 8 + T * 4
        ms_route = timed(lambda: M.moe_route(cfg, d["h"], wts["w_gate"], wts["logit_bias"], tr["logits"],
                                             tr["topk_ids"], tr["topk_gates"], tr["margin"], stream=stream),
                         max(args.steps, 5), True)
        stages["route"] = {"us": ms_route * 1e3, "GB/s": route_bytes / (ms_route * 1e-3) / 1e9}
        align_bytes = R * 4 + R + p_max * 4 + n_blocks * 4
        if w.reroute_depth and w.cap_den:  # the reroute policy also reads each token's logits
            rexp = torch.empty(R, dtype=torch.int32, device=dev)
            ms_align = timed(lambda: M.moe_align_reroute(cfg, tr["topk_ids"], tr["logits"], rexp, tr["route_kept"],
                                                         tr["sorted_route_ids"], tr["block_expert"],
                                                         tr["expert_offsets"], tr["num_padded"], tr["stats"], aws,
                                                         stream=stream), max(args.steps, 5), True)
            stages["align_reroute"] = {"us": ms_align * 1e3, "rerouted": int(tr["stats"][N + M.STAT["rerouted"]]),
                                       "dropped": int(tr["stats"][N + M.STAT["dropped"]])}
        else:
            ms_align = timed(lambda: M.moe_align(cfg, tr["topk_ids"], tr["route_kept"], tr["sorted_route_ids"],
                                                 tr["block_expert"], tr["expert_offsets"], tr["num_padded"],
                                                 tr["stats"], aws, stream=stream), max(args.steps, 5), True)
            stages["align"] = {"us": ms_align * 1e3, "GB/s": align_bytes / (ms_align * 1e-3) / 1e9}
        comb_bytes = kept_routes * H * asz + T * H * asz * 2 + R * 5
        ms_comb = timed(lambda: M.moe_combine(cfg, tr["y_route"], tr["topk_gates"], tr["route_kept"], None,
                                              d["residual"], out, stream=stream), max(args.steps, 5), True)
        stages["combine"] = {"us": ms_comb * 1e3, "GB/s": comb_bytes / (ms_comb * 1e-3) / 1e9}
        for name, ms_stage, nbytes in (("route", fwd_stage_ms[0], route_bytes),
                                       ("align" if "align" in stages else "align_reroute", fwd_stage_ms[1],
                                        align_bytes),
                                       ("combine", fwd_stage_ms[5], comb_bytes)):
            stages[name]["in_forward_us"] = ms_stage * 1e3
            stages[name]["in_forward_GB/s"] = nbytes / (ms_stage * 1e-3) / 1e9
        # router replay: the whole layer on the recorded ids of the forward above
        ms_replay = timed(lambda: M.moe_forward_replay(cfg, wts, d["h"], d["residual"], tr["topk_ids"], out, None, ws,
                                                       stream=stream), max(args.steps, 5), False)
        stages["forward_replay"] = {"us": ms_replay * 1e3, "tokens/s": T / (ms_replay * 1e-3)}
        for kname, v in stages.items():
            log(f"[bench] stage {kname}: " + ", ".join(f"{a} {b:,.2f}" for a, b in v.items()))

    # the stage events themselves cost time: the sum of the stages equals the fully
    # instrumented forward (first to last event), and that one is compared with the timed
    # step (which records events at the GEMM boundaries only)
    reconcile = {"stages_sum_us": round(sum(fwd_stage_ms) * 1e3, 2),
                 "instrumented_forward_us": round(fwd_events_ms * 1e3, 2),
                 "timed_step_us": round(ms * 1e3, 2),
                 "event_overhead_pct": round(100.0 * (fwd_events_ms - ms) / ms, 2),
                 "timed_step_gemm_us": {"gate_up_gemm": round(timed_gemm_ms[0] * 1e3, 2),
                                        "down_gemm": round(timed_gemm_ms[1] * 1e3, 2)},
                 "instrumented_gemm_us": {"gate_up_gemm": round(fwd_stage_ms[2] * 1e3, 2),
                                          "down_gemm": round(fwd_stage_ms[3] * 1e3, 2)}}
    log(f"[bench] stage sum {reconcile['stages_sum_us']:.1f} us, instrumented forward "
        f"{reconcile['instrumented_forward_us']:.1f} us, timed step {reconcile['timed_step_us']:.1f} us; "
        f"W13 {fwd_stage_ms[2] * 1e3:.1f} us instrumented vs {timed_gemm_ms[0] * 1e3:.1f} us in the timed steps")
    clocks = gemm_clock_report(cfg, wts, d, out, ws, stream, {"gate_up_gemm": ms_gate_up, "down_gemm": ms_down})
    log("[bench] shader clock inside the GEMMs (core cycles / wall clock per workgroup): "
        + ", ".join(f"{k} {v}" for k, v in clocks.items()))
    if not args.no_stages:
        smu = gfx_clock_report(step, tr, cfg, d, wts, act_t, stream)
        if smu:
            clocks["smu_gfxclk_MHz"] = {k: (v or {}).get("median") for k, v in smu.items()}
            log("[bench] SMU-reported gfx clock level (MHz, sampled while each runs back to back): "
                + ", ".join(f"{k} {v}" for k, v in smu.items()))

    achieved = stages["gate_up_gemm"]["TFLOP/s"]
    roofline = {"kernel": "ffn_gemm_bf16<W13+SwiGLU>", "bound": "mfma", "achieved": round(achieved, 2),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": _traffic(w.name, 1.0), "avg_launch_us": round(ms_gate_up * 1e3, 2),
                "flops_per_launch": gate_up_flops}

    ceil = None if args.no_stages else ceilings(stream)
    if ceil:
        log("[bench] measured ceilings: " + ", ".join(f"{a} {b:,.1f}" for a, b in ceil.items()))

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, d, args.cpu_sample)

    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16" if w.act_dtype == W.BF16 else "f32",
        "data": "synthetic (seeded; Gaussian inits; see DESIGN.md)",
        "config": {"workload": w.name, "T": w.T, "H": w.H, "N": w.N, "k": w.k, "I": w.I, "B": w.B,
                   "expert_dtype": w.expert_dtype, "capacity": None if w.cap_den == 0 else f"{w.cap_num}/{w.cap_den}",
                   "routing": w.routing, "n_shared": w.n_shared, "kept_routes": kept_routes,
                   "parallelism": "none (1 GPU)"},
        "roofline": roofline, "stages": {k: {a: round(b, 3) for a, b in v.items()} for k, v in stages.items()},
        "stage_reconciliation": reconcile, "sclk_MHz": clocks,
        "measured_ceilings": ceil,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


def ceilings(stream):
    """Measured ceilings on this GPU (libmoe_ceiling.so): 1 GiB copy and read streams,
    and back-to-back bf16 MFMAs from registers at one and two waves per SIMD."""
    import ctypes

    import torch

    from top_routing_expert_router_amd.build import CEILING_LIB_PATH

    L = ctypes.CDLL(CEILING_LIB_PATH)
    P, SZ, I32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32
    L.moe_ceiling_copy.argtypes, L.moe_ceiling_copy.restype = [P, P, SZ, P], I32
    L.moe_ceiling_read.argtypes, L.moe_ceiling_read.restype = [P, SZ, P, P], I32
    L.moe_ceiling_mfma_bf16.argtypes, L.moe_ceiling_mfma_bf16.restype = [I32, I32, P, P], I32
    sp = stream.cuda_stream
    nbytes = 1 << 30
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(4096, dtype=torch.float32, device="cuda")

    def time_ms(fn, reps=5):
        assert fn() == 0
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            assert fn() == 0
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    out = {}
    ms = time_ms(lambda: L.moe_ceiling_copy(src.data_ptr(), dst.data_ptr(), nbytes, sp))
    out["hbm_copy_GB/s"] = 2 * nbytes / (ms * 1e-3) / 1e9
    ms = time_ms(lambda: L.moe_ceiling_read(src.data_ptr(), nbytes, sink.data_ptr(), sp))
    out["hbm_read_GB/s"] = nbytes / (ms * 1e-3) / 1e9
    iters = 20000
    for wpe in (1, 2):
        ms = time_ms(lambda: L.moe_ceiling_mfma_bf16(iters, wpe, sink.data_ptr(), sp), reps=3)
        flops = 256 * 4 * wpe * iters * 8 * 32768.0
        out[f"mfma_bf16_TFLOP/s_{wpe}wave"] = flops / (ms * 1e-3) / 1e12
    del src, dst
    return {k: round(v, 1) for k, v in out.items()}


class GfxClockSampler:
    """The GPU's graphics (shader) clock as the SMU reports it (amdsmi GPU metrics, per XCD),
    sampled from a host thread every ~2 ms while a workload runs back to back."""

    def __init__(self):
        import amdsmi
        import torch
        self.a = amdsmi
        amdsmi.amdsmi_init()
        hs = amdsmi.amdsmi_get_processor_handles()
        self.h = hs[0]
        if len(hs) > 1:  # the handle whose PCI address is torch's device 0
            p = torch.cuda.get_device_properties(0)
            want = (getattr(p, "pci_domain_id", 0), getattr(p, "pci_bus_id", -1), getattr(p, "pci_device_id", 0))
            for h in hs:
                bdf = amdsmi.amdsmi_get_gpu_device_bdf(h)  # "dddd:bb:dd.f"
                dom, bus, rest = bdf.split(":")
                if (int(dom, 16), int(bus, 16), int(rest.split(".")[0], 16)) == want:
                    self.h = h
        self.sample()

    def sample(self):
        m = self.a.amdsmi_get_gpu_metrics_info(self.h)
        v = [c for c in (m.get("current_gfxclks") or []) if isinstance(c, (int, float)) and 0 < c < 10000]
        if not v and isinstance(m.get("current_gfxclk"), (int, float)):
            v = [m["current_gfxclk"]]
        return sum(v) / len(v) if v else None

    def during(self, fn, seconds: float = 0.6, batch: int = 8):
        import statistics
        import threading

        import torch
        got, stop = [], threading.Event()

        def loop():
            while not stop.is_set():
                try:
                    c = self.sample()
                except Exception:  # pragma: no cover - reported as missing
                    c = None
                if c:
                    got.append((time.perf_counter(), c))
                time.sleep(0.002)

        for _ in range(batch):
            fn()
        torch.cuda.synchronize()
        th = threading.Thread(target=loop, daemon=True)
        t0 = time.perf_counter()
        th.start()
        while time.perf_counter() - t0 < seconds:
            for _ in range(batch):
                fn()
            torch.cuda.synchronize()
        t1 = time.perf_counter()
        stop.set()
        th.join()
        # leave out the first tenth (the clock settling) and anything after the work ended
        vals = [c for t, c in got if t0 + 0.1 * (t1 - t0) <= t <= t1]
        if not vals:
            return None
        return {"median": round(statistics.median(vals)), "min": round(min(vals)), "max": round(max(vals)),
                "samples": len(vals)}


def ceiling_reader(buf, sink, stream):
    """A callable that enqueues the streaming read of buf (libmoe_ceiling.so) on stream."""
    import ctypes

    from top_routing_expert_router_amd.build import CEILING_LIB_PATH
    L = ctypes.CDLL(CEILING_LIB_PATH)
    L.moe_ceiling_read.argtypes, L.moe_ceiling_read.restype = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                                              ctypes.c_void_p], ctypes.c_int32
    n, p, q, sp = buf.numel() * buf.element_size(), buf.data_ptr(), sink.data_ptr(), stream.cuda_stream

    def go():
        assert L.moe_ceiling_read(p, n, q, sp) == 0
    return go


def clock_rates():
    """(wall-clock counter rate, peak shader clock) of the current device, in kHz."""
    import ctypes

    from top_routing_expert_router_amd.build import CEILING_LIB_PATH
    L = ctypes.CDLL(CEILING_LIB_PATH)
    wall, peak = ctypes.c_int32(), ctypes.c_int32()
    assert L.moe_ceiling_clock_rates(ctypes.byref(wall), ctypes.byref(peak)) == 0
    return wall.value, peak.value


def gemm_clock_report(cfg, wts, d, out, ws, stream, stage_ms):
    """The shader clock the routed expert GEMMs ran at inside one forward: each persistent
    workgroup's core-cycle and wall-clock counters at its start and end (moe_trace.gemm_clocks);
    clock = sum of cycles / sum of wall time over the workgroups.  The span from the first
    start to the last end, in wall-clock time, is given beside the stage's event time."""
    import numpy as np
    import torch

    import top_routing_expert_router_amd as M
    wall_khz, peak_khz = clock_rates()
    clk = torch.zeros(2 * M.CLOCK_SLOTS * 4, dtype=torch.int64, device="cuda")
    M.moe_forward(cfg, wts, d["h"], d["residual"], out, {"gemm_clocks": clk}, ws, stream=stream)
    torch.cuda.synchronize()
    c = clk.view(2, M.CLOCK_SLOTS, 4).cpu().numpy().astype(np.float64)
    res = {"peak_MHz": peak_khz / 1e3, "wall_clock_MHz": wall_khz / 1e3}
    for i, name in enumerate(("gate_up_gemm", "down_gemm")):
        x = c[i]
        used = x[:, 3] > x[:, 1]
        if not used.any():
            continue
        cyc, wall = x[used, 2] - x[used, 0], x[used, 3] - x[used, 1]
        per = cyc / wall * wall_khz / 1e3
        res[name] = {"MHz": round(float(cyc.sum() / wall.sum() * wall_khz / 1e3), 1),
                     "per_workgroup_MHz_min": round(float(per.min()), 1),
                     "per_workgroup_MHz_max": round(float(per.max()), 1), "workgroups": int(used.sum()),
                     "span_us": round(float((x[used, 3].max() - x[used, 1].min()) / wall_khz * 1e3), 1),
                     "event_us": round(stage_ms[name] * 1e3, 1)}
    return res


def gfx_clock_report(step, tr, cfg, d, wts, act_t, stream):
    """Sustained shader clock during the whole forward and during each expert GEMM alone (the
    standalone entry points, run back to back), or None where the SMU metrics are unreadable."""
    import top_routing_expert_router_amd as M
    try:
        smp = GfxClockSampler()
    except Exception as e:  # pragma: no cover - depends on the box
        log(f"[bench] shader clock unavailable: {e}")
        return None
    y = tr["y_route"]
    out = {}
    try:
        out["forward"] = smp.during(step)
        out["gate_up_gemm"] = smp.during(lambda: M.moe_expert_gate_up(
            cfg, d["h"], tr["sorted_route_ids"], tr["expert_offsets"], wts["w13"], wts.get("w13_scale"), tr["act"],
            None, stream=stream))
        out["down_gemm"] = smp.during(lambda: M.moe_expert_down(
            cfg, tr["act"], tr["sorted_route_ids"], tr["expert_offsets"], wts["w2"], wts.get("w2_scale"), y,
            stream=stream))
    except Exception as e:  # pragma: no cover
        log(f"[bench] shader clock sampling failed: {e}")
    return out or None


def host_cpu() -> dict:
    """The host's CPU model and core counts (lscpu, else /proc/cpuinfo)."""
    import subprocess
    info = {"model": None, "logical_cpus": os.cpu_count(), "physical_cores": None,
            "affinity_cpus": len(os.sched_getaffinity(0))}
    try:
        txt = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        kv = {a.strip(): b.strip() for a, _, b in (l.partition(":") for l in txt.splitlines())}
        info["model"] = kv.get("Model name")
        if kv.get("Core(s) per socket") and kv.get("Socket(s)"):
            info["physical_cores"] = int(kv["Core(s) per socket"]) * int(kv["Socket(s)"])
    except Exception:
        pass
    if info["model"] is None:
        try:
            for line in open("/proc/cpuinfo"):
                if line.startswith("model name"):
                    info["model"] = line.split(":", 1)[1].strip()
                    break
        except OSError:
            pass
    return info


def ec_stages(stages, w, cfg, d, wts, tr, out, ws, C, p_max, n_blocks, asz, timed, reps, stream):
    """Per-stage timings of an expert-choice layer (scores + picks, picks alone, alignment, combine)."""
    import top_routing_expert_router_amd as M

    T, H, N = w.T, w.H, w.N
    tn = T * N * 4
    # projection reads h and W_g; writes logits, scores, slots; picks and margins are small
    route_bytes = T * H * asz + N * H * asz + 3 * tn + N * C * 4
    f = lambda flags: M.moe_route_expert_choice(cfg, d["h"], wts["w_gate"], wts["logit_bias"], tr["logits"],
                                               tr["scores"], tr["choice_tokens"], tr["choice_slot"],
                                               tr["choice_margin"], flags=flags, stream=stream)
    ms = timed(lambda: f(0), reps, True)
    stages["route_expert_choice"] = {"us": ms * 1e3, "GB/s": route_bytes / (ms * 1e-3) / 1e9}
    # from given logits: the softmax pass (logits in, scores out) and the per-expert select
    # (each expert's score column in, its slot column out)
    ms = timed(lambda: f(M.MOE_ROUTE_LOGITS_IN), reps, True)
    stages["scores_and_picks"] = {"us": ms * 1e3, "GB/s": (4 * tn + N * C * 4) / (ms * 1e-3) / 1e9}
    ms = timed(lambda: M.moe_align_expert_choice(cfg, tr["choice_tokens"], tr["choice_slot"], tr["sorted_route_ids"],
                                                 tr["block_expert"], tr["expert_offsets"], tr["num_padded"],
                                                 tr["stats"], stream=stream), reps, True)
    stages["align_expert_choice"] = {"us": ms * 1e3, "GB/s": (N * C * 4 + tn + p_max * 4 + n_blocks * 4) / (ms * 1e-3) / 1e9,
                                     "unpicked": int(tr["stats"][N + M.STAT["unpicked"]]),
                                     "max_picks": int(tr["stats"][N + M.STAT["max_picks"]])}
    comb_bytes = N * C * H * asz + 2 * T * H * asz + 2 * tn
    ms = timed(lambda: M.moe_combine_expert_choice(cfg, tr["y_route"], tr["scores"], tr["choice_slot"], None,
                                                   d["residual"], out, stream=stream), reps, True)
    stages["combine"] = {"us": ms * 1e3, "GB/s": comb_bytes / (ms * 1e-3) / 1e9}


def cpu_baseline(w, d, sample: int, runs: int = 3):
    """The oracle (fp64 numpy) on this workload, restricted to a seeded token sample: the
    median of ``runs`` timed runs on the same host copies of the inputs."""
    import numpy as np
    import torch

    from oracle import moe_oracle as O

    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover - informational only
        threads = 1
    bits = lambda t: t.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16)
    log(f"[bench] cpu baseline: copying inputs to the host")
    h_b, wg_b = bits(d["h"]), bits(d["w_gate"])
    w13_b = d["w13"].to("cpu")
    w2_b = d["w2"].to("cpu")
    import workloads as W

    fp8 = w.expert_dtype == W.FP8
    if fp8:
        s13 = d["w13_scale"].float().cpu().double().numpy()
        s2 = d["w2_scale"].float().cpu().double().numpy()
    bias = None if d.get("bias") is None else d["bias"].double().cpu().numpy()
    sample = w.T if sample <= 0 else min(sample, w.T)
    g = torch.Generator().manual_seed(1234)
    tokens = torch.randperm(w.T, generator=g)[:sample].sort().values.numpy()
    times = []
    for _ in range(runs):
        t0 = time.perf_counter()
        res = _oracle_run(O, w, h_b, wg_b, w13_b, w2_b, s13 if fp8 else None, s2 if fp8 else None, fp8, bias, d,
                          tokens)
        times.append(time.perf_counter() - t0)
        assert res["out"].shape[0] == sample
    import statistics
    dt = statistics.median(times)
    log(f"[bench] cpu baseline: {sample} tokens, runs {' '.join(f'{t:.2f}' for t in times)} s")
    cpu = host_cpu()
    return {"value": round(sample / dt, 3), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "threads": int(threads), "cpu_model": cpu["model"], "host_logical_cpus": cpu["logical_cpus"],
            "host_physical_cores": cpu["physical_cores"], "affinity_cpus": cpu["affinity_cpus"],
            "runs_s": [round(t, 3) for t in times], "seconds": round(dt, 3),
            "sample": f"median of {runs} runs; {sample} seeded tokens of the {w.T}-token batch: full routing, "
                      f"capacity and alignment of all tokens, expert FFN (all experts' weights decoded to fp64) "
                      f"and combine for the sampled tokens; 'cores' = BLAS threads the oracle's matrix "
                      f"products ran on"}


def _oracle_run(O, w, h_b, wg_b, w13_b, w2_b, s13, s2, fp8, bias, d, tokens):
    """One oracle pass over the sampled tokens (decoding the stored inputs included)."""
    import numpy as np
    import torch
    h64 = O.decode_bf16(h_b)

    def expert(t, sc):
        if fp8:
            return lambda e: O.dequantize_blocks(t[e].numpy(), sc[e], w.scale_block)
        return lambda e: O.decode_bf16(t[e].view(torch.int16).numpy().view(np.uint16))

    shared = {}
    if w.n_shared:
        for which in ("w13", "w2"):
            t = d["shared_" + which].to("cpu")
            if fp8:
                sc = d[f"shared_{which}_scale"].float().cpu().double().numpy()
                shared["shared_" + which] = O.dequantize_blocks(t.numpy(), sc, w.scale_block)
            else:
                shared["shared_" + which] = O.decode_bf16(t.view(torch.int16).numpy().view(np.uint16))
    if w.routing == "expert_choice":
        res = O.expert_choice_forward(h64, O.decode_bf16(wg_b), expert(w13_b, s13 if fp8 else None),
                                      expert(w2_b, s2 if fp8 else None), k=w.k, B=w.B, cap_num=w.cap_num,
                                      cap_den=w.cap_den, residual=h64, tokens=tokens, bias=bias, **shared)
    else:
        res = O.moe_forward(h64, O.decode_bf16(wg_b), expert(w13_b, s13 if fp8 else None),
                            expert(w2_b, s2 if fp8 else None), k=w.k, B=w.B, cap_num=w.cap_num, cap_den=w.cap_den,
                            residual=h64, tokens=tokens, bias=bias, reroute_depth=w.reroute_depth, **shared)
    return res


if __name__ == "__main__":
    sys.exit(main())
