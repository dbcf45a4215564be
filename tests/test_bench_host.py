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
