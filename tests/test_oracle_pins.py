"""Pins for the CPU oracle: checks against what the pages and mathematics fix.

Nothing here compares the oracle with itself.  Each test uses a hand-worked
fixture under tests/golden/ (with its citation), brute force on tiny inputs,
a closed form, an invariant, or a library routine the step reduces to.
"""
import itertools
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import moe_oracle as O
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_fixture(name):
    d = {}
    cases = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, _, val = line.partition(":")
            if key == "case":
                cases.append(line[len("case:"):])
            else:
                d[key.strip()] = val.strip()
    return d, cases


def _floats(s):
    return np.array([float(x) for x in s.split()], dtype=np.float64)


def _ints(s):
    return np.array([int(x) for x in s.split()], dtype=np.int64)


# ------------------------------------------------------------------ decoding

def test_decode_e4m3_all_256_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = O.decode_e4m3(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    m = ~np.isnan(ref)
    assert np.array_equal(ours[m], ref[m])
    assert np.nanmax(ours) == 448.0 and np.count_nonzero(np.isnan(ours)) == 2


def test_decode_bf16_matches_torch():
    g = torch.Generator().manual_seed(1)
    x = torch.randn(4096, generator=g) * 1e3
    b = x.to(torch.bfloat16)
    ours = O.decode_bf16(b.view(torch.int16).numpy().view(np.uint16))
    assert np.array_equal(ours, b.to(torch.float64).numpy())


def test_round_bf16_matches_torch_cast_on_fp32_values():
    g = torch.Generator().manual_seed(11)
    x = torch.cat([torch.randn(20000, generator=g) * 10 ** float(p) for p in range(-6, 7)])
    # include exact ties: values halfway between two bf16 neighbours
    b = x.to(torch.bfloat16)
    up = (b.view(torch.int16) + 1).view(torch.bfloat16).float()  # next bf16 away from zero
    mid = (b.float() + up) / 2                                     # exact in fp32: a rounding tie
    assert torch.all(mid != b.float())
    for v in (x, mid):
        ours = O.round_bf16(v.double().numpy())
        ref = v.to(torch.bfloat16).double().numpy()
        assert np.array_equal(ours, ref)


def test_dequantize_blocks_hand_fixture():
    d, _ = _read_fixture("fp8_blocks.txt")
    blk = int(d["block"])
    codes = np.array([[int(c, 16) for c in row.split()] for row in d["codes"].split("|")], np.uint8)
    scales = np.array([[float(c) for c in row.split()] for row in d["scales"].split("|")])
    want = np.array([[float(c) for c in row.split()] for row in d["w"].split("|")])
    assert np.array_equal(O.dequantize_blocks(codes, scales, blk), want)


def test_fp8_generator_roundtrip_within_e4m3_step():
    # The workload encoder plus the oracle decoder reproduce the fp32 weights to within
    # half an e4m3 step (2^-4 relative) of each block's scale.
    wl = W.DEEPSEEKV3_FP8.with_(H=256, I=128)
    wf = W._expert_f32(wl, "w13", 3, "cpu")
    codes, scales = W.quantize_fp8_blocks(wf, 128)
    s = O.decode_bf16(scales.view(torch.int16).numpy().view(np.uint16))
    w = O.dequantize_blocks(codes.numpy(), s, 128)
    err = np.abs(w - wf.double().numpy())
    bound = np.repeat(np.repeat(s, 128, 0), 128, 1) * 448 * 2.0 ** -4
    assert np.all(err <= bound * 1.0001)


# ------------------------------------------------------------------ routing

def test_router_logits_against_library_linear():
    g = torch.Generator().manual_seed(2)
    h = torch.randn(17, 40, generator=g, dtype=torch.float64)
    wg = torch.randn(6, 40, generator=g, dtype=torch.float64)
    bias = torch.randn(6, generator=g, dtype=torch.float64)
    ref = F.linear(h, wg, bias).numpy()
    assert np.allclose(O.router_logits(h.numpy(), wg.numpy(), bias.numpy()), ref, rtol=1e-13, atol=1e-13)
    ref0 = torch.nn.Linear(40, 6, bias=False).double()
    with torch.no_grad():
        ref0.weight.copy_(wg)
        want = ref0(h).numpy()
    assert np.allclose(O.router_logits(h.numpy(), wg.numpy()), want, rtol=1e-13, atol=1e-13)


def _beats(la, a, lb, b):
    """Pairwise rule: does expert a rank above expert b?"""
    na, nb = math.isnan(la), math.isnan(lb)
    if na or nb:
        if na and nb:
            return a < b
        return nb
    if la != lb:
        return la > lb
    return a < b


def _brute_rank(row):
    N = len(row)
    wins = [sum(_beats(row[a], a, row[b], b) for b in range(N) if b != a) for a in range(N)]
    order = [None] * N
    for a, w in enumerate(wins):
        order[N - 1 - w] = a
    return order


def test_rank_experts_brute_force_with_ties_zeros_and_nan():
    alphabet = [-1.0, 0.0, -0.0, 1.0, float("nan")]
    rng = np.random.default_rng(3)
    for N in range(1, 7):
        for _ in range(300):
            row = rng.choice(alphabet, size=N)
            order = O.rank_experts(row[None, :])[0].tolist()
            assert order == _brute_rank(row.tolist()), row


def test_topk_exhaustive_small_alphabet():
    # Every logit vector over a 3-value alphabet for N = 5: the selected set dominates
    # every outsider under the pairwise rule, and is listed in rank order.
    N = 5
    for vals in itertools.product([0.0, 1.0, 2.0], repeat=N):
        row = np.array(vals)
        for k in range(1, N + 1):
            ids, _, margin = O.topk_route(row[None, :], k)
            ids = ids[0].tolist()
            assert len(set(ids)) == k
            out = [e for e in range(N) if e not in ids]
            for a in ids:
                for b in out:
                    assert _beats(row[a], a, row[b], b)
            for a, b in zip(ids, ids[1:]):
                assert _beats(row[a], a, row[b], b)
            if k < N:
                assert margin[0] == row[ids[-1]] - max(row[b] for b in out)
            else:
                assert margin[0] == np.inf


def test_topk_matches_torch_topk_on_tie_free_inputs():
    g = torch.Generator().manual_seed(4)
    l = torch.randn(500, 64, generator=g, dtype=torch.float64)
    for k in (1, 2, 8):
        ids, _, _ = O.topk_route(l.numpy(), k)
        ref = torch.topk(l, k, dim=1, largest=True, sorted=True).indices.numpy()
        assert np.array_equal(ids, ref)
        # selecting on softmax probabilities (the pages' worked router) gives the same experts
        ref_p = torch.topk(torch.softmax(l, dim=1), k, dim=1).indices.numpy()
        assert np.array_equal(ids, ref_p)


def test_golden_margin_and_gates_k4():
    d, _ = _read_fixture("router_margin_k4.txt")
    l = _floats(d["logits"])[None, :]
    ids, gates, margin = O.topk_route(l, int(d["k"]))
    assert ids[0].tolist() == _ints(d["ids"]).tolist()
    assert abs(margin[0] - float(d["margin"])) < 1e-15
    ratio = np.exp(_floats(d["gate_ratio_exponents"]))
    assert np.allclose(gates[0] / gates[0][0], ratio, rtol=1e-14)
    assert abs(gates[0].sum() - 1.0) < 1e-15


def test_golden_tie_rule():
    _, cases = _read_fixture("tie_rule_k2.txt")
    assert len(cases) == 5
    for c in cases:
        lg, ids, mg = [p.split(":")[-1].strip() for p in c.split("|")]
        l = np.array([float(x) for x in lg.split()])[None, :]
        got_ids, _, got_m = O.topk_route(l, 2)
        assert got_ids[0].tolist() == [int(x) for x in ids.split()], c
        want_m = float(mg)
        assert (math.isnan(want_m) and math.isnan(got_m[0])) or got_m[0] == want_m, c


def test_gates_identities():
    g = torch.Generator().manual_seed(5)
    l = (torch.randn(300, 16, generator=g, dtype=torch.float64) * 3).numpy()
    for k in (1, 2, 4, 16):
        ids, gates, _ = O.topk_route(l, k)
        assert np.allclose(gates.sum(1), 1.0, atol=1e-14)
        if k == 1:
            assert np.all(gates == 1.0)
        if k == 16:  # N = k: renormalised gates are the full softmax (library routine)
            p = torch.softmax(torch.from_numpy(l), dim=1).numpy()
            assert np.allclose(gates, np.take_along_axis(p, ids, 1), rtol=1e-13)
        sel = np.take_along_axis(l, ids, 1)
        # softmax over the selected logits alone (library) -- equal to softmax-then-renorm
        ref = torch.softmax(torch.from_numpy(sel), dim=1).numpy()
        assert np.allclose(gates, ref, rtol=1e-12, atol=1e-15)
        # gates are non-increasing in rank (larger logit, larger gate)
        assert np.all(np.diff(gates, axis=1) <= 1e-15)
    # without renormalisation the gates are plain softmax probabilities of the selected experts
    ids, gates, _ = O.topk_route(l, 2, renormalize=False)
    p = torch.softmax(torch.from_numpy(l), dim=1).numpy()
    assert np.allclose(gates, np.take_along_axis(p, ids, 1), rtol=1e-13)


# ------------------------------------------------------------------ capacity, alignment, stats

def test_capacity_formulas():
    # Switch-style: tokens / experts x factor, k = 1 (2048 / 16 x 1.25 = 160)
    assert O.capacity(2048, 1, 16, 5, 4) == 160
    assert O.capacity(64, 2, 8, 0, 0) is None
    # The worked example's int(mean(load) x 1.25) with load = bincount of the flattened ids
    for seed in range(5):
        ids = W.random_routes(96, 8, 2, seed).long()
        load = torch.bincount(ids.flatten(), minlength=8)
        assert O.capacity(96, 2, 8, 5, 4) == int(load.double().mean() * 1.25)
    assert O.capacity(3, 1, 8, 5, 4) == 0  # small batch: literal formula gives zero


def _brute_fill(ids_flat, N, cap):
    """A dispatcher that walks tokens in batch order and appends each route to its
    expert's buffer while the buffer has room."""
    buffers = {e: [] for e in range(N)}
    kept = []
    for r, e in enumerate(ids_flat):
        if len(buffers[e]) < cap:
            buffers[e].append(r)
            kept.append(True)
        else:
            kept.append(False)
    return np.array(kept), buffers


def test_capacity_keep_brute_force_and_identities():
    for T, N, k in itertools.product(range(1, 7), range(1, 4), range(1, 3)):
        if k > N:
            continue
        rng = np.random.default_rng(T * 100 + N * 10 + k)
        for _ in range(20):
            ids = np.stack([rng.permutation(N)[:k] for _ in range(T)])
            for cap in range(0, T * k + 2):
                kept = O.capacity_keep(ids, N, cap)
                want, _ = _brute_fill(ids.reshape(-1).tolist(), N, cap)
                assert np.array_equal(kept, want)
                load = torch.bincount(torch.from_numpy(ids).flatten(), minlength=N)
                dropped = int((load - cap).clamp(min=0).sum())
                assert dropped == kept.size - kept.sum()
            assert O.capacity_keep(ids, N, None).all()
            assert not O.capacity_keep(ids, N, 0).any()


def test_capacity_keep_invalid_ids_never_kept():
    ids = np.array([[0, 5], [-1, 1], [2, 2]])
    kept = O.capacity_keep(ids, 3, None)
    assert kept.tolist() == [True, False, False, True, True, True]


def _brute_align(ids_flat, kept, N, B):
    R = len(ids_flat)
    keys = sorted((ids_flat[r], r) for r in range(R) if kept[r])
    seq, blocks, offs = [], [], [0]
    for e in range(N):
        mem = [r for (ee, r) in keys if ee == e]
        pad = (-len(mem)) % B
        seq += mem + [R] * pad
        blocks += [e] * ((len(mem) + pad) // B)
        offs.append(len(seq))
    return seq, blocks, offs


def test_align_golden_fixture():
    d, _ = _read_fixture("align_capacity_T4_k2_N3_B2.txt")
    T, k, N, B = (int(d[x]) for x in "TkNB")
    ids = _ints(d["ids"]).reshape(T, k)
    for tag, cap in (("dropless", None), ("cf1", O.capacity(T, k, N, 1, 1))):
        if tag == "cf1":
            assert cap == int(d["cf1.cap"])
        kept = O.capacity_keep(ids, N, cap)
        assert kept.astype(int).tolist() == _ints(d[tag + ".kept"]).tolist()
        al = O.align(ids, kept, N, B)
        assert al["sorted_route_ids"].tolist() == _ints(d[tag + ".sorted_route_ids"]).tolist()
        assert al["block_expert"].tolist() == _ints(d[tag + ".block_expert"]).tolist()
        assert al["expert_offsets"].tolist() == _ints(d[tag + ".expert_offsets"]).tolist()
        assert al["num_padded"] == int(d[tag + ".num_padded"])
    st = O.routing_stats(ids, O.capacity_keep(ids, N, 2), N, 2)
    assert st["load"].tolist() == _ints(d["load"]).tolist()
    assert st["dropped_tokens"] == int(d["cf1.dropped"])
    assert st["max_expert_load"] == int(d["cf1.max_expert_load"])
    assert st["min_expert_load"] == int(d["cf1.min_expert_load"])
    assert st["imbalance_ratio"] == float(d["cf1.imbalance_ratio"])
    assert st["drop_fraction"] == float(d["cf1.drop_fraction"])


def test_align_brute_force_and_invariants():
    for seed in range(60):
        rng = np.random.default_rng(seed)
        T, N = int(rng.integers(1, 20)), int(rng.integers(1, 9))
        k = int(rng.integers(1, N + 1))
        B = int(rng.choice([1, 2, 4, 8]))
        ids = np.stack([rng.permutation(N)[:k] for _ in range(T)])
        cap = None if seed % 3 == 0 else int(rng.integers(0, T + 1))
        kept = O.capacity_keep(ids, N, cap)
        al = O.align(ids, kept, N, B)
        seq, blocks, offs = _brute_align(ids.reshape(-1).tolist(), kept, N, B)
        R = T * k
        sr = al["sorted_route_ids"]
        assert sr.shape[0] == R + N * (B - 1)
        assert sr[:len(seq)].tolist() == seq and np.all(sr[len(seq):] == R)
        assert al["block_expert"][:len(blocks)].tolist() == blocks
        assert np.all(al["block_expert"][len(blocks):] == -1)
        assert al["expert_offsets"].tolist() == offs and al["num_padded"] == offs[-1]
        # invariants: a permutation of the kept routes, homogeneous blocks, counts = bincount
        valid = sr[sr != R]
        assert sorted(valid.tolist()) == np.nonzero(kept)[0].tolist()
        flat = ids.reshape(-1)
        for b, e in enumerate(al["block_expert"].tolist()):
            rows = sr[b * B:(b + 1) * B]
            rows = rows[rows != R]
            assert e >= 0 or rows.size == 0
            assert np.all(flat[rows] == e)
        cnt = np.bincount(flat[kept], minlength=N)
        assert np.array_equal(np.diff(al["expert_offsets"]), -(-cnt // B) * B)


# ------------------------------------------------------------------ expert FFN and combine

def test_silu_against_library():
    x = np.concatenate([np.linspace(-800, 800, 4001), np.linspace(-6, 6, 1001)])
    ref = F.silu(torch.from_numpy(x)).numpy()
    assert np.allclose(O.silu(x), ref, rtol=1e-15, atol=1e-300)


def test_w13_projection_and_activation_against_library():
    # [W1 x ; W3 x] is F.linear with the stacked weight; the activation is F.silu of the gate
    # half times the up half; W2 applied to it is the whole expert (swiglu_expert, pinned
    # below against an independent torch FFN).  H != I so that a transposed operand fails.
    g = torch.Generator().manual_seed(12)
    M, H, I = 7, 24, 40
    x = torch.randn(M, H, generator=g, dtype=torch.float64)
    w13 = torch.randn(2 * I, H, generator=g, dtype=torch.float64) / math.sqrt(H)
    w2 = torch.randn(H, I, generator=g, dtype=torch.float64) / math.sqrt(I)
    u = O.w13_projection(x.numpy(), w13.numpy())
    assert u.shape == (M, 2 * I)
    assert np.allclose(u[:, :I], F.linear(x, w13[:I]).numpy(), rtol=1e-14, atol=1e-14)
    assert np.allclose(u[:, I:], F.linear(x, w13[I:]).numpy(), rtol=1e-14, atol=1e-14)
    a = O.swiglu_activation(x.numpy(), w13.numpy())
    want = F.silu(F.linear(x, w13[:I])) * F.linear(x, w13[I:])
    assert a.shape == (M, I) and np.allclose(a, want.numpy(), rtol=1e-14, atol=1e-14)
    assert np.allclose(a @ w2.numpy().T, O.swiglu_expert(x.numpy(), w13.numpy(), w2.numpy()), rtol=1e-13, atol=1e-13)


def _torch_swiglu(x, w13, w2):
    I = w13.shape[0] // 2
    gate, up = w13[:I], w13[I:]
    return F.linear(F.silu(F.linear(x, gate)) * F.linear(x, up), w2)


def test_single_expert_top1_is_a_plain_swiglu_ffn():
    # N = 1, k = 1: the layer is h + FFN(h) (gate exactly 1)
    g = torch.Generator().manual_seed(6)
    T, H, I = 9, 24, 40  # H != I so that a transposed operand cannot pass
    h = torch.randn(T, H, generator=g, dtype=torch.float64)
    wg = torch.randn(1, H, generator=g, dtype=torch.float64)
    w13 = torch.randn(1, 2 * I, H, generator=g, dtype=torch.float64) / math.sqrt(H)
    w2 = torch.randn(1, H, I, generator=g, dtype=torch.float64) / math.sqrt(I)
    res = O.moe_forward(h.numpy(), wg.numpy(), lambda e: w13[e].numpy(), lambda e: w2[e].numpy(),
                        k=1, B=4, residual=h.numpy())
    want = (h + _torch_swiglu(h, w13[0], w2[0])).numpy()
    assert np.allclose(res["out"], want, rtol=1e-12, atol=1e-12)
    res0 = O.moe_forward(h.numpy(), wg.numpy(), lambda e: w13[e].numpy(), lambda e: w2[e].numpy(), k=1, B=4)
    assert np.allclose(res0["out"], _torch_swiglu(h, w13[0], w2[0]).numpy(), rtol=1e-12, atol=1e-12)


def _torch_dense_mixture(h, wg, w13, w2, k):
    """Independent layer: softmax router, torch.topk on probabilities, renormalise, loop experts."""
    probs = torch.softmax(F.linear(h, wg), dim=-1)
    gv, gi = probs.topk(k, dim=-1)
    gv = gv / gv.sum(-1, keepdim=True)
    out = h.clone()
    for e in range(wg.shape[0]):
        y = _torch_swiglu(h, w13[e], w2[e])
        wgt = (gv * (gi == e)).sum(-1, keepdim=True)
        out = out + wgt * y
    return out


def test_all_experts_selected_is_a_dense_soft_mixture():
    g = torch.Generator().manual_seed(7)
    T, H, I, N = 11, 16, 20, 4
    h = torch.randn(T, H, generator=g, dtype=torch.float64)
    wg = torch.randn(N, H, generator=g, dtype=torch.float64)
    w13 = torch.randn(N, 2 * I, H, generator=g, dtype=torch.float64) / 4
    w2 = torch.randn(N, H, I, generator=g, dtype=torch.float64) / 4
    res = O.moe_forward(h.numpy(), wg.numpy(), lambda e: w13[e].numpy(), lambda e: w2[e].numpy(),
                        k=N, B=2, residual=h.numpy())
    p = torch.softmax(F.linear(h, wg), -1)
    want = h + sum(p[:, e:e + 1] * _torch_swiglu(h, w13[e], w2[e]) for e in range(N))
    assert np.allclose(res["out"], want.numpy(), rtol=1e-12, atol=1e-12)


def test_toy_layer_against_independent_torch_layer():
    wl = W.TOY_FP32
    d = W.layer_inputs(wl)
    h = d["h"].double()
    wg, w13, w2 = d["w_gate"].double(), d["w13"].double(), d["w2"].double()
    res = O.moe_forward(h.numpy(), wg.numpy(), lambda e: w13[e].numpy(), lambda e: w2[e].numpy(),
                        k=wl.k, B=wl.B, residual=h.numpy())
    want = _torch_dense_mixture(h, wg, w13, w2, wl.k).numpy()
    rel = np.abs(res["out"] - want).max() / np.abs(want).max()
    assert rel < 1e-12
    # the toy batch has no near-ties at fp64 precision, so the torch topk agrees on every route
    assert res["margin"].min() > 1e-9


def test_partial_and_full_drop_give_residual_plus_survivors():
    d, _ = _read_fixture("align_capacity_T4_k2_N3_B2.txt")
    T, k, N = 4, 2, 3
    ids = _ints(d["ids"]).reshape(T, k)
    g = torch.Generator().manual_seed(8)
    H, I = 6, 10
    h = torch.randn(T, H, generator=g, dtype=torch.float64)
    w13 = torch.randn(N, 2 * I, H, generator=g, dtype=torch.float64)
    w2 = torch.randn(N, H, I, generator=g, dtype=torch.float64)
    gates = np.array([[0.75, 0.25]] * T)
    kept = O.capacity_keep(ids, N, 2)   # r5 (t2, j1) and r7 (t3, j1) dropped
    y = O.expert_ffn(h.numpy(), ids, kept, lambda e: w13[e].numpy(), lambda e: w2[e].numpy(), N)
    out = O.combine(y, gates, kept, T, H, residual=h.numpy())
    for t in (2, 3):
        e0 = int(ids[t, 0])
        want = h[t] + 0.75 * _torch_swiglu(h[t:t + 1], w13[e0], w2[e0])[0]
        assert np.allclose(out[t], want.numpy(), rtol=1e-12, atol=1e-12)
    # capacity zero: every route dropped, each output row is exactly its residual row
    none = O.capacity_keep(ids, N, 0)
    out0 = O.combine({}, gates, none, T, H, residual=h.numpy())
    assert np.array_equal(out0, h.numpy())


def test_shared_expert_adds_a_dense_ffn():
    g = torch.Generator().manual_seed(9)
    T, H, I, N = 5, 8, 12, 3
    h = torch.randn(T, H, generator=g, dtype=torch.float64)
    wg = torch.randn(N, H, generator=g, dtype=torch.float64)
    w13 = torch.randn(N, 2 * I, H, generator=g, dtype=torch.float64)
    w2 = torch.randn(N, H, I, generator=g, dtype=torch.float64)
    s13 = torch.randn(2 * I, H, generator=g, dtype=torch.float64)
    s2 = torch.randn(H, I, generator=g, dtype=torch.float64)
    base = O.moe_forward(h.numpy(), wg.numpy(), lambda e: w13[e].numpy(), lambda e: w2[e].numpy(), k=2, B=2)
    withs = O.moe_forward(h.numpy(), wg.numpy(), lambda e: w13[e].numpy(), lambda e: w2[e].numpy(), k=2, B=2,
                          shared_w13=s13.numpy(), shared_w2=s2.numpy())
    assert np.allclose(withs["out"] - base["out"], _torch_swiglu(h, s13, s2).numpy(), rtol=1e-12, atol=1e-12)


def test_fresh_router_load_is_roughly_uniform():
    # The worked example: a fresh router on 4096 random 512-wide tokens, 8 experts, top-2.
    g = torch.Generator().manual_seed(10)
    h = torch.randn(4096, 512, generator=g, dtype=torch.float64)
    lin = torch.nn.Linear(512, 8, bias=False).double()
    torch.nn.init.normal_(lin.weight, 0.0, 0.02, generator=g)
    ids, _, _ = O.topk_route(O.router_logits(h.numpy(), lin.weight.detach().numpy()), 2)
    load = O.routing_stats(ids, np.ones(ids.size, bool), 8, None)["load"]
    assert load.sum() == 8192
    assert load.min() > 0.75 * 1024 and load.max() < 1.25 * 1024


def test_sampled_tokens_equal_full_pass():
    wl = W.TOY_FP32
    d = W.layer_inputs(wl)
    args = (d["h"].double().numpy(), d["w_gate"].double().numpy(),
            lambda e: d["w13"][e].double().numpy(), lambda e: d["w2"][e].double().numpy())
    full = O.moe_forward(*args, k=wl.k, B=wl.B, residual=d["h"].double().numpy())
    sub = np.array([3, 17, 40, 63])
    part = O.moe_forward(*args, k=wl.k, B=wl.B, residual=d["h"].double().numpy(), tokens=sub)
    # BLAS may block a smaller product differently: equal up to fp64 rounding
    assert np.allclose(part["out"], full["out"][sub], rtol=1e-13, atol=1e-13)


# ------------------------------------------------------------------ router replay

def test_golden_replay_k2():
    d, _ = _read_fixture("replay_k2.txt")
    l = _floats(d["logits"])[None, :]
    ids = _ints(d["replay_ids"])[None, :]
    gates, margin = O.replay_route(l, ids, renormalize=True)
    assert np.allclose(gates[0], _floats(d["gates"]), rtol=1e-14, atol=0)
    gates_sm, _ = O.replay_route(l, ids, renormalize=False)
    assert np.allclose(gates_sm[0], _floats(d["gates_softmax"]), rtol=1e-14, atol=0)
    assert margin[0] == float(d["margin"])


def test_replay_of_own_route_reproduces_it():
    rng = np.random.default_rng(5)
    for N, k in ((8, 2), (16, 1), (64, 8), (6, 6)):
        l = rng.standard_normal((40, N))
        l[3, :] = 0.25          # all tied
        l[4, 1] = np.nan
        for renorm in (True, False):
            ids, gates, margin = O.topk_route(l, k, renorm)
            g2, m2 = O.replay_route(l, ids, renorm)
            assert np.allclose(g2, gates, rtol=1e-15, atol=0)
            assert np.array_equal(m2, margin)


def test_replay_gates_follow_the_recorded_order_and_ignore_invalid_ids():
    rng = np.random.default_rng(6)
    N, k = 12, 4
    l = rng.standard_normal((30, N))
    ids = np.stack([rng.permutation(N)[:k] for _ in range(30)])
    g, _ = O.replay_route(l, ids)
    perm = np.array([2, 0, 3, 1])
    gp, _ = O.replay_route(l, ids[:, perm])
    assert np.allclose(gp, g[:, perm], rtol=1e-15, atol=0)
    assert np.allclose(g.sum(axis=1), 1.0, rtol=0, atol=1e-15)
    # ids outside [0, N) carry no weight; the rest renormalise among themselves
    bad = ids.copy()
    bad[:, 1] = N
    bad[:, 3] = -1
    gb, _ = O.replay_route(l, bad)
    assert np.all(gb[:, [1, 3]] == 0)
    ref, _ = O.replay_route(l, ids[:, [0, 2]])
    assert np.allclose(gb[:, [0, 2]], ref, rtol=1e-15, atol=0)
    # one recorded expert: gate exactly 1
    g1, _ = O.replay_route(l, ids[:, :1])
    assert np.all(g1 == 1.0)


def test_forward_replay_of_own_ids_matches_forward():
    w = W.TOY_FP32
    d = W.layer_inputs(w, device="cpu")
    f64 = lambda t: t.double().numpy()
    w13 = f64(d["w13"]); w2 = f64(d["w2"])
    kw = dict(k=w.k, B=w.B, residual=f64(d["residual"]))
    a = O.moe_forward(f64(d["h"]), f64(d["w_gate"]), lambda e: w13[e], lambda e: w2[e], **kw)
    b = O.moe_forward(f64(d["h"]), f64(d["w_gate"]), lambda e: w13[e], lambda e: w2[e], replay_ids=a["ids"], **kw)
    assert np.array_equal(a["out"], b["out"]) and np.array_equal(a["gates"], b["gates"])
    # a different recorded route changes the experts that run, not the projection
    other = np.roll(a["ids"], 1, axis=1)
    c = O.moe_forward(f64(d["h"]), f64(d["w_gate"]), lambda e: w13[e], lambda e: w2[e], replay_ids=other, **kw)
    assert np.array_equal(c["ids"], other) and np.array_equal(c["logits"], a["logits"])
    assert np.allclose(c["gates"], np.roll(a["gates"], 1, axis=1), rtol=1e-15, atol=0)


# ------------------------------------------------------------------ reroute overflow policy

def test_golden_reroute():
    d, _ = _read_fixture("reroute_T6_N3_k1.txt")
    T, N, k, cap = int(d["T"]), int(d["N"]), int(d["k"]), int(d["cap"])
    l = _floats(d["logits"]).reshape(T, N)
    assert O.capacity(T, k, N, 1, 1) == cap
    ids, _, _ = O.topk_route(l, k)
    for depth in (0, 1, 2, 5):
        expert, kept, rerouted = O.capacity_reroute(ids, l, N, cap, depth)
        want = _ints(d[f"expert_depth{min(depth, 2)}"])
        assert expert.tolist() == want.tolist(), depth
        assert kept.tolist() == (want >= 0).tolist()
        assert rerouted.tolist() == ((want >= 0) & (want != ids.reshape(-1))).tolist()


def _reroute_by_rounds(ids, logits, N, cap, depth):
    """The same policy written round-parallel: per round, gather every token's request,
    then per expert admit the first `room` requests in token order."""
    T, k = ids.shape
    kept = O.capacity_keep(ids, N, cap)
    expert = np.where(kept, ids.reshape(-1), -1)
    room = np.array([cap - np.count_nonzero(expert == e) for e in range(N)])
    order = O.rank_experts(logits)
    offered = np.zeros((T, N), dtype=bool)
    for t in range(T):
        offered[t, [e for e in ids[t] if 0 <= e < N]] = True
    for _ in range(depth):
        req = []
        for t in range(T):
            pend = [j for j in range(k) if not kept[t * k + j] and 0 <= ids[t, j] < N]
            free = [e for e in order[t] if not offered[t, e]]
            if pend and free:
                offered[t, free[0]] = True
                req.append((t, pend[0], free[0]))
        for e in range(N):
            mine = [(t, j) for t, j, c in req if c == e]
            for t, j in mine[: max(room[e], 0)]:
                kept[t * k + j] = True
                expert[t * k + j] = e
            room[e] -= min(len(mine), max(room[e], 0))
    return expert, kept


def test_reroute_invariants_and_round_parallel_form():
    rng = np.random.default_rng(9)
    for trial in range(60):
        N = int(rng.integers(2, 9))
        k = int(rng.integers(1, min(N, 3) + 1))
        T = int(rng.integers(1, 30))
        l = rng.standard_normal((T, N))
        l[rng.random((T, N)) < 0.1] = 0.5                # ties
        ids, _, _ = O.topk_route(l, k)
        if trial % 3 == 0:                                # replayed, non-top-k ids (some invalid)
            ids = np.stack([rng.permutation(N)[:k] for _ in range(T)])
            ids[rng.random((T, k)) < 0.1] = N
        cap = int(rng.integers(0, 4))
        base = O.capacity_keep(ids, N, cap)
        prev = base
        for depth in range(0, N - k + 2):
            expert, kept, rerouted = O.capacity_reroute(ids, l, N, cap, depth)
            ex2, kept2 = _reroute_by_rounds(ids, l, N, cap, depth)
            assert np.array_equal(expert, ex2) and np.array_equal(kept, kept2)
            assert np.all(kept[base]) and np.array_equal(expert[base], ids.reshape(-1)[base])  # phase 1 stays
            assert np.all(kept[prev])                                                         # monotone in depth
            assert np.array_equal(rerouted, kept & ~base)
            load = np.bincount(expert[kept], minlength=N)
            assert np.all(load <= cap)
            for t in range(T):
                mine = expert[t * k:(t + 1) * k][kept[t * k:(t + 1) * k]]
                assert len(set(mine.tolist())) == len(mine)               # no expert twice per token
                rr = expert[t * k:(t + 1) * k][rerouted[t * k:(t + 1) * k]]
                assert not set(rr.tolist()) & set(ids[t].tolist())         # reroutes leave the recorded set
            if depth == 0:
                assert np.array_equal(kept, base)
            prev = kept
    # no capacity: nothing overflows, nothing reroutes
    l = rng.standard_normal((10, 4))
    ids, _, _ = O.topk_route(l, 2)
    e, kp, rr = O.capacity_reroute(ids, l, 4, None, 3)
    assert kp.all() and not rr.any()


def test_forward_reroute_runs_the_new_expert_with_the_old_gate():
    # Switch-like: top-1, tight capacity; a rerouted token's output is h + 1 * E_c(h)
    rng = np.random.default_rng(3)
    T, H, I, N, k = 12, 8, 16, 3, 1
    h = rng.standard_normal((T, H))
    wg = rng.standard_normal((N, H))
    w13 = rng.standard_normal((N, 2 * I, H)) / math.sqrt(H)
    w2 = rng.standard_normal((N, H, I)) / math.sqrt(I)
    kw = dict(k=k, B=2, cap_num=1, cap_den=1, residual=h)
    drop = O.moe_forward(h, wg, lambda e: w13[e], lambda e: w2[e], **kw)
    rr = O.moe_forward(h, wg, lambda e: w13[e], lambda e: w2[e], reroute_depth=N - k, **kw)
    assert rr["stats"]["rerouted"] > 0
    for t in range(T):
        if rr["rerouted"][t]:
            c = rr["run_ids"][t, 0]
            assert c != drop["ids"][t, 0] and not drop["kept"][t]
            assert np.allclose(rr["out"][t], h[t] + O.swiglu_expert(h[t:t + 1], w13[c], w2[c])[0], rtol=1e-13)
        elif drop["kept"][t]:
            assert np.array_equal(rr["out"][t], drop["out"][t])


# ------------------------------------------------------------------ expert-choice routing

def test_golden_expert_choice():
    d, _ = _read_fixture("expert_choice_T6_N3.txt")
    T, N, k = int(d["T"]), int(d["N"]), int(d["k"])
    S = _floats(d["scores"]).reshape(T, N)
    assert O.expert_choice_capacity(T, k, N, 1, 1) == int(d["C_cf1"])
    assert O.expert_choice_capacity(T, k, N, 0, 0) == int(d["C_cf1"])  # unset factor = 1
    assert O.expert_choice_capacity(T, k, N, 3, 2) == int(d["C_cf3_2"])
    for C in (2, 3):
        tokens, slot, margin = O.expert_choice_select(S, C)
        assert tokens.reshape(-1).tolist() == _ints(d[f"picks_C{C}"]).tolist()
        assert margin.tolist() == _floats(d[f"margin_C{C}"]).tolist()
        assert np.count_nonzero(slot >= 0, axis=1).tolist() == _ints(d[f"picks_per_token_C{C}"]).tolist()
        for e in range(N):
            assert [slot[t, e] for t in tokens[e]] == list(range(C))


def _beats(sa, a, sb, b):
    """(score sa, token a) ranks above (score sb, token b): larger score, then lower index; NaN last."""
    na, nb = math.isnan(sa), math.isnan(sb)
    if na or nb:
        return (a < b) if (na and nb) else nb
    return sa > sb or (sa == sb and a < b)


def test_expert_choice_select_brute_force():
    # every C-subset of tokens: exactly one dominates all the others under the order
    # (score desc, lower token first, NaN last), and it is the oracle's pick
    rng = np.random.default_rng(21)
    for trial in range(150):
        T, N = int(rng.integers(1, 7)), int(rng.integers(1, 4))
        S = rng.choice(np.array([0.0, 0.25, 0.5, -0.0, np.nan]) if trial % 5 == 0 else np.array([0.1, 0.2, 0.7]),
                       size=(T, N))
        for C in range(0, T + 1):
            tokens, slot, margin = O.expert_choice_select(S, C)
            for e in range(N):
                good = [set(P) for P in itertools.combinations(range(T), C)
                        if all(_beats(S[p, e], p, S[q, e], q) for p in P for q in range(T) if q not in P)]
                assert len(good) == 1 and set(tokens[e].tolist()) == good[0]
                assert tokens[e].tolist() == sorted(tokens[e].tolist())
                assert [t for t in range(T) if slot[t, e] >= 0] == tokens[e].tolist()
                if 0 < C < T:
                    vals = sorted(S[:, e], key=lambda v: (not math.isnan(v), v), reverse=True)
                    assert (np.isnan(margin[e]) and (math.isnan(vals[C - 1]) or math.isnan(vals[C]))) or \
                        margin[e] == vals[C - 1] - vals[C]
                else:
                    assert margin[e] == np.inf


def test_expert_choice_select_matches_torch_topk_on_distinct_scores():
    g = torch.Generator().manual_seed(4)
    for T, N, C in ((50, 4, 7), (300, 16, 60), (1000, 8, 250)):
        S = torch.rand(T, N, generator=g, dtype=torch.float64)
        tokens, _, margin = O.expert_choice_select(S.numpy(), C)
        vals, idx = torch.topk(S, C + 1, dim=0)
        for e in range(N):
            assert sorted(idx[:C, e].tolist()) == tokens[e].tolist()
            assert margin[e] == (vals[C - 1, e] - vals[C, e]).item()


def test_expert_scores_closed_forms_and_softmax():
    # logits ln(w) -> scores w / sum(w); NaN weighs zero; rows sum to one; torch's softmax
    w = np.array([[1.0, 1.0, 2.0], [6.0, 1.0, 1.0], [1.0, 3.0, 4.0]])
    S = O.expert_scores(np.log(w))
    assert np.allclose(S, w / w.sum(axis=1, keepdims=True), rtol=1e-15, atol=0)
    l = np.array([[0.0, np.nan, np.log(3.0)]])
    assert np.allclose(O.expert_scores(l), [[0.25, 0.0, 0.75]], rtol=1e-15, atol=0)
    rng = np.random.default_rng(2)
    l = rng.standard_normal((200, 37)) * 3
    S = O.expert_scores(l)
    assert np.allclose(S.sum(axis=1), 1.0, rtol=0, atol=1e-14)
    assert np.allclose(S, torch.softmax(torch.from_numpy(l), dim=1).numpy(), rtol=1e-14, atol=0)
    # the scores of a token's top-k experts are its token-choice gates without renormalisation
    ids, gates, _ = O.topk_route(l, 5, renormalize=False)
    assert np.array_equal(np.take_along_axis(S, ids, axis=1), gates)


def test_expert_choice_capacity_formula():
    assert O.expert_choice_capacity(4096, 2, 8, 0, 0) == 1024      # Mixtral-shaped, factor 1
    assert O.expert_choice_capacity(2048, 1, 16, 5, 4) == 160      # the Switch capacity, factor 1.25
    assert O.expert_choice_capacity(5, 1, 8, 1, 1) == 0            # fewer tokens than experts
    assert O.expert_choice_capacity(10, 2, 4, 4, 2) == 10          # factor N/k: every expert takes every token
    assert O.expert_choice_capacity(10, 2, 4, 9, 1) == 10          # never more than T


def test_expert_choice_align_invariants():
    rng = np.random.default_rng(5)
    for T, N, C, B in ((9, 3, 4, 2), (40, 5, 13, 8), (7, 2, 7, 16), (6, 4, 0, 8)):
        S = rng.random((T, N))
        tokens, _, _ = O.expert_choice_select(S, C)
        al = O.expert_choice_align(tokens, T, B)
        Cp = -(-C // B) * B
        assert al["segment"] == Cp and al["num_padded"] == N * Cp
        assert al["expert_offsets"].tolist() == [e * Cp for e in range(N + 1)]
        assert al["block_expert"].tolist() == [b // (Cp // B) for b in range(N * Cp // B)] if Cp else \
            al["block_expert"].size == 0
        for e in range(N):
            seg = al["sorted_tokens"][e * Cp:(e + 1) * Cp]
            assert seg[:C].tolist() == tokens[e].tolist() and np.all(seg[C:] == T)


def test_golden_expert_choice_align():
    d, _ = _read_fixture("expert_choice_align_T6_N3.txt")
    T, N = int(d["T"]), int(d["N"])
    for C, B in ((2, 4), (2, 8), (3, 2), (3, 3)):
        tokens = _ints(d[f"picks_C{C}"]).reshape(N, C)
        al = O.expert_choice_align(tokens, T, B)
        tag = f"B{B}_C{C}"
        assert al["sorted_tokens"].tolist() == _ints(d[tag + ".sorted"]).tolist(), tag
        assert al["block_expert"].tolist() == _ints(d[tag + ".blocks"]).tolist(), tag
        assert al["expert_offsets"].tolist() == _ints(d[tag + ".offsets"]).tolist(), tag
        assert al["num_padded"] == int(d[tag + ".num_padded"]), tag


def test_expert_choice_align_equals_token_choice_align_of_the_picks():
    # The picks written as a token-choice route list: route r = e*C + j runs expert e and
    # carries token tokens[e, j].  The token-choice alignment (pinned by brute force above)
    # groups routes by expert in ascending route id, i.e. ascending token within an expert,
    # and pads every expert's C routes to Cp rows, so its segments are the expert-choice
    # segments with route ids in place of tokens.
    rng = np.random.default_rng(11)
    for T, N, C, B in ((9, 3, 4, 2), (40, 5, 13, 8), (7, 2, 7, 16), (64, 8, 16, 8), (33, 6, 1, 4), (6, 4, 0, 8)):
        S = rng.random((T, N))
        tokens, _, _ = O.expert_choice_select(S, C)
        ec = O.expert_choice_align(tokens, T, B)
        routes = np.repeat(np.arange(N), C)               # expert of route r = e*C + j
        tc = O.align(routes.reshape(-1, 1), np.ones(N * C, bool), N, B)
        P = ec["num_padded"]
        assert tc["num_padded"] == P
        assert tc["expert_offsets"].tolist() == ec["expert_offsets"].tolist()
        assert tc["block_expert"][:P // B].tolist() == ec["block_expert"].tolist()
        assert np.all(tc["block_expert"][P // B:] == -1)
        r = tc["sorted_route_ids"][:P]
        real = r < N * C
        as_tokens = np.where(real, tokens.reshape(-1)[np.minimum(r, max(N * C - 1, 0))] if N * C else T, T)
        assert as_tokens.tolist() == ec["sorted_tokens"].tolist()


def _ec_layer(seed, T, H, I, N):
    rng = np.random.default_rng(seed)
    h = rng.standard_normal((T, H))
    wg = rng.standard_normal((N, H)) * 0.3
    w13 = rng.standard_normal((N, 2 * I, H)) / math.sqrt(H)
    w2 = rng.standard_normal((N, H, I)) / math.sqrt(I)
    return h, wg, w13, w2


def test_expert_choice_with_every_token_is_the_dense_soft_mixture():
    # C = T (factor N/k): every expert takes every token with weight softmax_e -- the same
    # layer as token choice with k = N and no renormalisation (a different, pinned path)
    T, H, I, N, k = 9, 8, 12, 4, 2
    h, wg, w13, w2 = _ec_layer(1, T, H, I, N)
    ec = O.expert_choice_forward(h, wg, lambda e: w13[e], lambda e: w2[e], k=k, B=4, cap_num=N, cap_den=k,
                                 residual=h)
    assert ec["cap"] == T and ec["stats"]["unpicked_tokens"] == 0 and ec["stats"]["max_picks"] == N
    tc = O.moe_forward(h, wg, lambda e: w13[e], lambda e: w2[e], k=N, B=4, renormalize=False, residual=h)
    assert np.allclose(ec["out"], tc["out"], rtol=1e-12, atol=1e-12)


def test_expert_choice_single_expert_is_a_plain_swiglu_ffn():
    T, H, I = 7, 8, 12
    h, wg, w13, w2 = _ec_layer(2, T, H, I, 1)
    ec = O.expert_choice_forward(h, wg, lambda e: w13[e], lambda e: w2[e], k=1, B=4, residual=h)
    assert ec["cap"] == T and np.all(ec["scores"] == 1.0)
    x = torch.from_numpy(h)
    ref = x + F.linear(F.silu(F.linear(x, torch.from_numpy(w13[0, :I]))) * F.linear(x, torch.from_numpy(w13[0, I:])),
                       torch.from_numpy(w2[0]))
    assert np.allclose(ec["out"], ref.numpy(), rtol=1e-13, atol=1e-13)


def test_expert_choice_forward_picks_and_unpicked_tokens():
    T, H, I, N, k = 16, 8, 12, 4, 1
    h, wg, w13, w2 = _ec_layer(3, T, H, I, N)
    ec = O.expert_choice_forward(h, wg, lambda e: w13[e], lambda e: w2[e], k=k, B=2, residual=h)
    C = ec["cap"]
    assert C == 4
    picks = np.count_nonzero(ec["slot"] >= 0, axis=1)
    assert ec["stats"]["unpicked_tokens"] == np.count_nonzero(picks == 0) > 0
    assert picks.sum() == N * C
    for t in range(T):
        want = h[t].copy()
        for e in range(N):
            if ec["slot"][t, e] >= 0:
                want = want + ec["scores"][t, e] * O.swiglu_expert(h[t:t + 1], w13[e], w2[e])[0]
        if picks[t] == 0:
            assert np.array_equal(ec["out"][t], h[t])       # the dual failure: h alone
        assert np.allclose(ec["out"][t], want, rtol=1e-13, atol=1e-13)
    # a sample of rows gives the same rows (up to the matrix product's blocking)
    sub = O.expert_choice_forward(h, wg, lambda e: w13[e], lambda e: w2[e], k=k, B=2, residual=h, tokens=[3, 0, 11])
    assert np.allclose(sub["out"], ec["out"][[3, 0, 11]], rtol=1e-14, atol=1e-14)
