"""Tile modes of the grouped down-projection GEMM give the same bits.

On the Mixtral-shaped layer the down projection makes one to four rounds of 256x256
tiles over the CUs, so an expert's last m-tile of at most 128 rows runs as micro tiles
(up to 64 rows x 64 weight rows, 128-deep stages in a four-buffer ring: four of them for
a last m-tile of up to 64 rows, eight for 65 to 128), scheduled after the full-height
tiles.  Every output element is still one MFMA chain over K in ascending 16-wide steps,
so each y row must equal, bit for bit, the same row computed in a problem small enough
that no micro tile is used (one expert's rows in identity mode: full, half or quarter
tiles).
"""
import sys

import numpy as np
import pytest
import torch

import top_routing_expert_router_amd as M

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


@pytest.mark.parametrize("I", [14336, 768, 256])
def test_w2_micro_tiles_match_standard_tiles(I):
    # I = 14336: 112 stages of 128 (whole groups of four); 768: six (the last group has
    # two); 256: two (no stage issued from inside the ring)
    T, H, N, k, B = 4096, 4096, 8, 2, 64
    # expert loads: last m-tiles of 64 (expert 1) and 128 rows (expert 2) become four and
    # eight micro tiles per weight n-tile; 1000 and 952 leave padded, partly empty last tiles of 256 and 192 rows
    loads = [1024, 1088, 1152, 1024, 1000, 1000, 952, 952]
    assert sum(loads) == T * k
    _say("w2 micro tiles vs standard tiles, I", I, "loads", loads)
    g = torch.Generator().manual_seed(5)
    perm = torch.randperm(T * k, generator=g).numpy()
    cfg = M.make_config(T, H, N, k, I, B)
    p_max, _ = M.moe_align_sizes(cfg)
    sorted_ids = np.full(p_max, T * k, dtype=np.int32)
    offsets = np.zeros(N + 1, dtype=np.int32)
    pos = 0
    for e, n in enumerate(loads):
        offsets[e] = sum(-(-x // B) * B for x in loads[:e])
        sorted_ids[offsets[e]:offsets[e] + n] = np.sort(perm[pos:pos + n])
        pos += n
    offsets[N] = sum(-(-x // B) * B for x in loads)
    gd = torch.Generator(device=DEV).manual_seed(6)
    act = (torch.randn(p_max, I, device=DEV, generator=gd) * 0.05).to(torch.bfloat16)
    w2 = (torch.randn(N, H, I, device=DEV, generator=gd) / I ** 0.5).to(torch.bfloat16)
    y = torch.full((T * k, H), 7.0, dtype=torch.bfloat16, device=DEV)
    sd = torch.from_numpy(sorted_ids).to(DEV)
    od = torch.from_numpy(offsets).to(DEV)
    M.moe_expert_down(cfg, act, sd, od, w2, None, y)
    torch.cuda.synchronize()
    checked = 0
    for e, n in enumerate(loads):
        seg = -(-n // B) * B
        # one expert's padded rows alone, identity rows: at most 5 x 16 tiles, no micro tiles
        ce = M.make_config(seg, H, 1, 1, I, B)
        ye = torch.empty(seg, H, dtype=torch.bfloat16, device=DEV)
        M.moe_expert_down(ce, act[offsets[e]:offsets[e] + seg].contiguous(), None, None, w2[e:e + 1].contiguous(),
                          None, ye)
        torch.cuda.synchronize()
        routes = torch.from_numpy(sorted_ids[offsets[e]:offsets[e] + n].astype(np.int64)).to(DEV)
        got = y[routes].view(torch.int16)
        want = ye[:n].view(torch.int16)
        bad = (got != want).any(dim=1).nonzero().flatten()
        assert bad.numel() == 0, (e, bad[:8].tolist())
        checked += n
    assert checked == T * k  # every y row (all filled with 7.0 before) was compared
    _say(f"  {checked} y rows bitwise equal to the standard-tile results")


def test_w2_micro_tiles_identity_rows():
    """Identity rows (no routing: the shared-expert form) with micro tiles: T = 4160 tokens
    make 17 x 16 down-projection tiles, so the last m-tile (64 rows) runs as micro tiles;
    every y row must equal, bit for bit, the same row computed in two smaller calls whose
    tiles do not use them (2048 and 2112 tokens: 128 and 144 tiles)."""
    T, H, I = 4160, 4096, 14336
    cfg = M.make_config(T, H, 1, 1, I, 64)
    gd = torch.Generator(device=DEV).manual_seed(11)
    act = (torch.randn(T, I, device=DEV, generator=gd) * 0.05).to(torch.bfloat16)
    w2 = (torch.randn(1, H, I, device=DEV, generator=gd) / I ** 0.5).to(torch.bfloat16)
    y = torch.full((T, H), 7.0, dtype=torch.bfloat16, device=DEV)
    M.moe_expert_down(cfg, act, None, None, w2, None, y)
    parts = []
    for r0, r1 in ((0, 2048), (2048, T)):
        c = M.make_config(r1 - r0, H, 1, 1, I, 64)
        yp = torch.empty(r1 - r0, H, dtype=torch.bfloat16, device=DEV)
        M.moe_expert_down(c, act[r0:r1].contiguous(), None, None, w2, None, yp)
        parts.append(yp)
    torch.cuda.synchronize()
    want = torch.cat(parts)
    bad = (y.view(torch.int16) != want.view(torch.int16)).any(dim=1).nonzero().flatten()
    assert bad.numel() == 0, bad[:8].tolist()
    _say(f"  {T} identity y rows bitwise equal without micro tiles")


@pytest.mark.parametrize("name", ["toy_fp32", "mixtral_bf16", "mixtral_ec_bf16", "deepseekv3_fp8"])
def test_forward_stage_events(name):
    """Trace stage events: recorded in order on the forward's stream, the stage times add
    up to the whole, and recording them changes no output bit."""
    import workloads as W
    import harness as Hn
    w = {"toy_fp32": W.TOY_FP32, "mixtral_bf16": W.MIXTRAL_BF16.with_(T=512),
         "mixtral_ec_bf16": W.MIXTRAL_EC_BF16.with_(T=512),
         "deepseekv3_fp8": W.DEEPSEEKV3_FP8.with_(T=200, N=24, H=1024, I=512)}[name]
    _say("stage events", name)
    d = W.layer_inputs(w)
    dv = Hn.to_dev(d)
    out0, _ = Hn.run_forward(w, dv, trace=False)
    cfg = Hn.config(w)
    ws = torch.empty(M.moe_workspace_size(cfg, M.MOE_OP_FORWARD), dtype=torch.uint8, device=DEV)
    out = torch.empty_like(out0)
    wts = {k: dv.get(k) for k in Hn.WEIGHT_KEYS}
    wts["logit_bias"] = None if dv.get("bias") is None else dv["bias"].to(DEV)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(M.TRACE_EVENTS)]
    before, after = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for rep in range(2):
        before.record()
        M.moe_forward(cfg, wts, dv["h"], dv["h"], out, {"stage_events": evs}, ws)
        after.record()
        torch.cuda.synchronize()
        stages = [evs[i].elapsed_time(evs[i + 1]) for i in range(M.TRACE_EVENTS - 1)]
        assert all(t >= 0 for t in stages), stages
        total = evs[0].elapsed_time(evs[-1])
        assert abs(sum(stages) - total) <= 1e-3 + 1e-6 * total
        assert before.elapsed_time(evs[0]) >= 0 and evs[-1].elapsed_time(after) >= 0
        if w.n_shared == 0:
            assert stages[4] < 0.05  # no shared expert: an empty stage
        assert torch.equal(out.view(torch.int16 if out.element_size() == 2 else torch.int32),
                           out0.view(torch.int16 if out0.element_size() == 2 else torch.int32))
    _say("  stage ms", [round(t, 4) for t in stages])


def test_forward_timing_only_stage_events():
    """The bench's in-step GEMM events: HIP events created for timing only (no system-scope
    fence), passed as raw handles at the W13 and W2 boundaries with the other boundaries null.
    Recorded in order inside the forward (between ordinary events recorded just before and
    after it), the two GEMM times are positive and fit in the forward, and no output bit
    changes."""
    import bench
    import workloads as W
    import harness as Hn
    w = W.MIXTRAL_BF16.with_(T=512)
    d = W.layer_inputs(w)
    dv = Hn.to_dev(d)
    out0, _ = Hn.run_forward(w, dv, trace=False)
    cfg = Hn.config(w)
    ws = torch.empty(M.moe_workspace_size(cfg, M.MOE_OP_FORWARD), dtype=torch.uint8, device=DEV)
    out = torch.empty_like(out0)
    wts = {k: dv.get(k) for k in Hn.WEIGHT_KEYS}
    wts["logit_bias"] = None if dv.get("bias") is None else dv["bias"].to(DEV)
    ev = [bench.TimingEvent() for _ in range(3)]  # after the alignment, after W13, after W2
    before, after = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for rep in range(2):
        before.record()
        M.moe_forward(cfg, wts, dv["h"], dv["h"], out,
                      {"stage_events": [None, None] + [e.handle for e in ev] + [None, None]}, ws)
        after.record()
        torch.cuda.synchronize()
        w13, w2 = ev[0].elapsed_time(ev[1]), ev[1].elapsed_time(ev[2])
        whole = before.elapsed_time(after)
        assert 0 < w13 and 0 < w2 and w13 + w2 <= whole, (w13, w2, whole)
        assert torch.equal(out.view(torch.int16), out0.view(torch.int16))
    _say("  timing-only events: W13 %.4f ms, W2 %.4f ms of %.4f" % (w13, w2, whole))


@pytest.mark.parametrize("name", ["mixtral_bf16", "deepseekv3_fp8"])
def test_forward_gemm_clock_stamps(name):
    """Trace clock stamps of the routed W13 and W2 launches: every persistent workgroup of a
    launch writes its start and end counters (end after start, within the real span of the
    stage), the slots beyond the grid stay untouched, and stamping changes no output bit."""
    import workloads as W
    import harness as Hn
    w = {"mixtral_bf16": W.MIXTRAL_BF16.with_(T=1024),
         "deepseekv3_fp8": W.DEEPSEEKV3_FP8.with_(T=200, N=24, H=1024, I=512)}[name]
    _say("gemm clock stamps", name)
    d = W.layer_inputs(w)
    dv = Hn.to_dev(d)
    out0, _ = Hn.run_forward(w, dv, trace=False)
    cfg = Hn.config(w)
    ws = torch.empty(M.moe_workspace_size(cfg, M.MOE_OP_FORWARD), dtype=torch.uint8, device=DEV)
    out = torch.empty_like(out0)
    wts = {k: dv.get(k) for k in Hn.WEIGHT_KEYS}
    wts["logit_bias"] = None if dv.get("bias") is None else dv["bias"].to(DEV)
    clk = torch.full((2 * M.CLOCK_SLOTS * 4,), -1, dtype=torch.int64, device=DEV)
    M.moe_forward(cfg, wts, dv["h"], dv["h"], out, {"gemm_clocks": clk}, ws)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out0.view(torch.int16))
    c = clk.view(2, M.CLOCK_SLOTS, 4).cpu()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for i in range(2):
        used = c[i, :, 0] != -1
        n = int(used.sum())
        assert 8 <= n <= ((cus + 7) // 8) * 8 and bool(used[:n].all()), n  # slots 0..grid-1
        x = c[i, :n]
        assert bool((x[:, 2] >= x[:, 0]).all()) and bool((x[:, 3] >= x[:, 1]).all())
        assert bool((c[i, n:] == -1).all())
        mhz = float((x[:, 2] - x[:, 0]).sum()) / float((x[:, 3] - x[:, 1]).sum())
        _say(f"  launch {i}: {n} workgroups, core cycles per wall-clock tick {mhz:.2f}")
        assert 0.5 < mhz < 100  # a shader clock between 0.05 and 10 GHz against a 100 MHz wall clock


@pytest.mark.parametrize("expert_dtype", ["bf16", "fp8_e4m3"])
def test_routed_tiles_match_quarter_tiles(expert_dtype):
    """Experts of 1088, 1152, 448, 320, 576, 200 and 64 rows (full 256-row tiles followed by
    partly filled full, half and quarter tiles) give, for every act and y row, the same bits as
    the same rows computed 64 at a time in identity mode (quarter tiles only): every output
    element is one MFMA chain over K whatever the tile and mode it lands in."""
    import workloads as W
    import harness as Hn
    N, k, B = 8, 1, 64
    loads = [1088, 1152, 448, 320, 576, 200, 64, 0]
    T = sum(loads)
    base = W.MIXTRAL_BF16 if expert_dtype == "bf16" else W.DEEPSEEKV3_FP8
    w = base.with_(T=T, H=512, I=512, N=N, k=k, B=B, n_shared=0)
    _say("routed tiles vs quarter tiles", expert_dtype, loads)
    d = Hn.to_dev(W.layer_inputs(w))
    cfg = Hn.config(w)
    p_max, _ = M.moe_align_sizes(cfg)
    g = torch.Generator().manual_seed(9)
    perm = torch.randperm(T, generator=g).numpy()   # route r = token r (k = 1)
    sorted_ids = np.full(p_max, T, dtype=np.int32)
    offsets = np.zeros(N + 1, dtype=np.int32)
    pos = 0
    for e, n in enumerate(loads):
        offsets[e + 1] = offsets[e] + -(-n // B) * B
        sorted_ids[offsets[e]:offsets[e] + n] = np.sort(perm[pos:pos + n])
        pos += n
    sd, od = torch.from_numpy(sorted_ids).to(DEV), torch.from_numpy(offsets).to(DEV)
    act = torch.zeros(p_max, w.I, dtype=torch.bfloat16, device=DEV)
    y = torch.full((T, w.H), 7.0, dtype=torch.bfloat16, device=DEV)
    M.moe_expert_ffn(cfg, d["h"], sd, od, d["w13"], d["w2"], d.get("w13_scale"), d.get("w2_scale"), act, None, y)
    torch.cuda.synchronize()
    checked = 0
    for e, n in enumerate(loads):
        if n == 0:
            continue
        routes = torch.from_numpy(sorted_ids[offsets[e]:offsets[e] + n].astype(np.int64)).to(DEV)
        x = d["h"][routes].contiguous()
        sc13 = None if d.get("w13_scale") is None else d["w13_scale"][e:e + 1].contiguous()
        sc2 = None if d.get("w2_scale") is None else d["w2_scale"][e:e + 1].contiguous()
        for c0 in range(0, n, 64):  # 64 rows at a time: one quarter tile per call
            c1 = min(n, c0 + 64)
            ce = Hn.config(w, T=c1 - c0, N=1)
            ae = torch.empty(c1 - c0, w.I, dtype=torch.bfloat16, device=DEV)
            ye = torch.empty(c1 - c0, w.H, dtype=torch.bfloat16, device=DEV)
            M.moe_expert_ffn(ce, x[c0:c1].contiguous(), None, None, d["w13"][e:e + 1].contiguous(),
                             d["w2"][e:e + 1].contiguous(), sc13, sc2, ae, None, ye)
            torch.cuda.synchronize()
            assert torch.equal(act[offsets[e] + c0:offsets[e] + c1].view(torch.int16), ae.view(torch.int16)), (e, c0)
            assert torch.equal(y[routes[c0:c1]].view(torch.int16), ye.view(torch.int16)), (e, c0)
            checked += c1 - c0
    assert checked == T
    _say(f"  {checked} act and y rows bitwise equal to quarter-tile results")
