"""Host-side legs of bench.py that need no GPU: the CPU baseline on tiny shapes (every
expert dtype, the bias and the shared expert) and the counter/trace summaries."""
import os

import numpy as np

import bench
import workloads as W


def test_cpu_baseline_runs_on_every_weight_format():
    for w in (W.TOY_FP32.with_(expert_dtype=W.F32), W.SWITCH_REROUTE_BF16.with_(T=64, H=128, I=256),
              W.DEEPSEEKV3_FP8.with_(T=64, H=256, I=256, N=8, k=2),
              W.DEEPSEEKV3_EC_FP8.with_(T=64, H=256, I=256, N=8, k=2), W.MIXTRAL_EC_BF16.with_(T=64, H=128, I=256)):
        if w.act_dtype == W.F32:
            continue  # the baseline decodes bf16 activations (the bench workloads' format)
        d = W.layer_inputs(w, device="cpu")
        r = bench.cpu_baseline(w, d, 4)
        assert r["kind"] == "oracle" and r["value"] > 0 and np.isfinite(r["value"])


def test_summaries_read_rocprof_csv(tmp_path):
    fetch, write, trace = (tmp_path / n for n in ("f", "w", "t"))
    for d in (fetch, write, trace):
        os.makedirs(d)
    rows = [("copy16(x)", 1048576.0, 1048576.0), ("void ffn_gemm_bf16<0, false>(a)", 2000.0, 100.0),
            ("router_bf16<1>(x)", 10.0, 1.0)]
    hdr = '"Kernel_Name","Counter_Name","Counter_Value"\n'
    (fetch / "run_counter_collection.csv").write_text(hdr + "".join(f'"{n}","FETCH_SIZE",{f / 2}\n' for n, f, _ in rows))
    (write / "run_counter_collection.csv").write_text(hdr + "".join(f'"{n}","WRITE_SIZE",{v}\n' for n, _, v in rows))
    assert bench.summarize_counters(str(fetch), str(write), "unit_test", out_dir=str(tmp_path)) == 0
    import json
    dd = json.load(open(tmp_path / "gate_up_gemm_unit_test_traffic.json"))
    assert dd["fetch_scale"] == 2.0 and dd["write_scale"] == 1.0
    assert dd["hbm_bytes_per_launch"] == round(2000 * 1024 + 100 * 1024)
    (trace / "run_kernel_trace.csv").write_text(
        '"Kernel_Name","Start_Timestamp","End_Timestamp"\n"copy16(x)",0,1000\n"router_bf16<1>(x)",0,3000\n')
    assert bench.summarize_trace(str(trace), "unit_test") == 0


def test_trace_summary_timed_steps(tmp_path, capsys):
    """Timed-step launches are picked by dispatch order after the warmup ones; with a shared
    expert each forward's two GEMM launches are split into routed and shared."""
    rows, t = [], 0
    for fwd in range(5):  # 2 warmup, 2 timed, 1 after
        for name, dur in (("router_ring<256, 64, 3, 0>(x)", 10), ("void ffn_gemm_bf16<0, true>(a)", 1000 + fwd),
                          ("void ffn_gemm_bf16<1, true>(a)", 500), ("void ffn_gemm_bf16<0, true>(a)", 100 + fwd),
                          ("void ffn_gemm_bf16<1, true>(a)", 50), ("combine_rows<x>", 20)):
            rows.append(f'"{name}",{t},{t + dur * 1000}\n')
            t += dur * 1000 + 7
    rows.append(f'"topk_gates(x)",{t},{t + 4000}\n')  # a standalone launch, not part of each forward
    d = tmp_path / "t"
    os.makedirs(d)
    (d / "run_kernel_trace.csv").write_text('"Kernel_Name","Start_Timestamp","End_Timestamp"\n' + "".join(rows))
    assert bench.summarize_trace(str(d), "deepseekv3_fp8", warmup=2, steps=2) == 0
    out = capsys.readouterr().out
    everything, timed = out.split("# the 2 timed steps")
    def table(txt):
        t = {}
        for l in txt.splitlines():
            f = l.split()
            if not f or l.startswith("#") or f[0] == "kernel" or l.startswith(" "):
                continue
            key = f[0] + (" " + f[1] if len(f) > 1 and f[1].startswith("(") else "")
            t[key] = f[2:] if key.endswith(")") else f[1:]
        return t
    a, b = table(everything), table(timed)
    assert a["route_ring"][0] == "5" and a["gate_up_gemm"][0] == "10"
    assert b["gate_up_gemm (routed)"][:2] == ["2", "1002.50"] and b["gate_up_gemm (shared)"][:2] == ["2", "102.50"]
    assert b["route_ring"][:2] == ["2", "10.00"] and b["combine"][0] == "2"
    assert "route_topk" in a and "route_topk" not in b


def test_trace_summary_names_the_reroute_kernels(tmp_path, capsys):
    """The reroute policy's two kernels (the ranking, then the one-workgroup rounds) get
    stage names of their own in the trace summary."""
    d = tmp_path / "r"
    os.makedirs(d)
    (d / "run_kernel_trace.csv").write_text(
        '"Kernel_Name","Start_Timestamp","End_Timestamp"\n'
        '"void moe::(anonymous namespace)::reroute_rank<16>(float const*, int, int, unsigned char*)",0,4000\n'
        '"moe::(anonymous namespace)::reroute_capacity(int const*, unsigned char const*)",5000,65000\n')
    assert bench.summarize_trace(str(d), "switch_reroute_bf16") == 0
    out = capsys.readouterr().out
    names = {l.split()[0] for l in out.splitlines() if l and not l.startswith("#")}
    assert {"reroute_rank", "reroute"} <= names
