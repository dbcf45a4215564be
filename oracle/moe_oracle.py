"""CPU oracle for the MoE layer forward pass -- TEST INFRASTRUCTURE ONLY.

Token-choice routing (each token picks its top-k experts) with the drop and reroute
overflow policies and router replay, and expert-choice routing (each expert picks its
top-C tokens).

Only the tests, the smoke entry point and the CPU-baseline leg of the benchmark
may import this module.  The product path (the HIP library and its Python
binding) never calls it and shares no code with it.

Plain, slow, obviously correct: numpy in float64 on inputs decoded exactly,
one function per step of the layer, each citing the passage it follows.
Library primitives used as steps: matrix product, ``exp``, stable argsort.

Pages cited (by title, then section / figure):
  [R&R]  "Mixture-of-experts routing & LLM repeatability" (vincentschmalbach.com; no headings,
         cited by the paragraph's subject)
  [BI]   "Why temperature=0 Still Gives Different Answers: Batch Invariance"
  [RB]   "Route-Block Membership Selects Packed-AWQ Arithmetic"
  [MIR]  "Mixture-of-Experts Routing at Inference Time"

Readings taken where the pages are silent are marked READING and listed in the
design notes.  Parity status: every function here is pinned by tests under
``tests/`` marked ``not gpu`` (brute force, closed forms, library special
cases, hand-worked fixtures); no function is "parity unpinned".
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np

__all__ = [
    "decode_bf16", "decode_e4m3", "round_bf16", "dequantize_blocks", "router_logits", "rank_experts",
    "topk_route", "replay_route", "capacity", "capacity_keep", "capacity_reroute", "align", "silu", "swiglu_expert",
    "w13_projection", "swiglu_activation",
    "expert_ffn", "combine", "routing_stats", "moe_forward", "expert_scores", "expert_choice_capacity",
    "expert_choice_select", "expert_choice_align", "expert_choice_combine", "expert_choice_forward",
]


# ---------------------------------------------------------------- input decoding

def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64: the top 16 bits of an IEEE binary32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def decode_e4m3(codes: np.ndarray) -> np.ndarray:
    """OCP FP8 E4M3FN codes (uint8) -> float64, from the format's definition.

    sign = bit 7, exponent = bits 6..3 (bias 7), mantissa = bits 2..0.
    exponent 0: subnormal m * 2^-9;  exponent 15 with mantissa 7: NaN (no infinities);
    otherwise (1 + m/8) * 2^(exp-7).  Largest finite value 448.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    ex = (c >> 3) & 0xF
    man = c & 0x7
    val = np.where(ex == 0, man * 2.0 ** -9, (1.0 + man / 8.0) * np.exp2(ex - 7.0))
    val = np.where((ex == 15) & (man == 7), np.nan, val)
    return sign * val


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round to the nearest bfloat16 value (8 significant bits), ties to even.

    Diagnostic only: lets the oracle mimic a pipeline that stores intermediates
    in bf16, to tell rounding from defects when a tolerance is approached.
    Normal-range values only (no subnormal or overflow handling).
    """
    m, e = np.frexp(np.asarray(x, np.float64))
    return np.ldexp(np.round(m * 256.0) / 256.0, e)


def dequantize_blocks(codes: np.ndarray, scales: np.ndarray, block: int) -> np.ndarray:
    """w[r, c] = e4m3(codes[r, c]) * scale[r // block, c // block], exactly, in float64.

    READING: "per-128-block bf16 scales" means one scale per 128 x 128 tile of
    (output row, reduction column); ``scales`` is given already decoded (float64).
    """
    q = decode_e4m3(codes)
    s = np.repeat(np.repeat(np.asarray(scales, np.float64), block, axis=-2), block, axis=-1)
    return q * s


# ---------------------------------------------------------------- routing

def router_logits(h: np.ndarray, w_gate: np.ndarray, bias: Optional[np.ndarray] = None) -> np.ndarray:
    """One logit per expert: l[t, e] = sum_i h[t, i] * W_g[e, i] (+ bias[e]).

    [MIR] "How sparse routing works": the router is one learned matrix that
    projects h to N logits; the worked router is a bias-free linear layer whose
    weight is stored [N, hidden] ("Worked example: a top-k router").  The
    optional additive bias is the workload's per-expert logit offset.
    """
    l = np.asarray(h, np.float64) @ np.asarray(w_gate, np.float64).T
    if bias is not None:
        l = l + np.asarray(bias, np.float64)[None, :]
    return l


def rank_experts(logits: np.ndarray) -> np.ndarray:
    """Per token, all experts in rank order: logit descending, ties to the lower index.

    [R&R] paragraph on the top-k step: the choice is fixed once scores, tie rule
    and capacity rules are fixed.  READING: the tie rule is "lowest expert index
    wins"; comparison is IEEE (so -0 == +0); a NaN logit ranks below every
    number, NaNs among themselves by index.  Ranking is done on logits, which
    orders experts exactly as the (strictly monotone) softmax does.
    """
    l = np.asarray(logits, np.float64) + 0.0  # +0.0 turns -0 into +0
    # A stable ascending sort of -l puts the largest logit first, keeps equal
    # values in index order, and sends NaN to the end.
    return np.argsort(-l, axis=1, kind="stable")


def topk_route(logits: np.ndarray, k: int, renormalize: bool = True):
    """Top-k experts, their gates and the router margin, per token.

    Returns (ids [T, k] int64 in rank order, gates [T, k] float64, margin [T] float64).

    Gates follow [MIR] "How sparse routing works" and the worked TopKRouter:
    softmax over all N logits, keep the k selected, divide by their sum
    (renormalize); without renormalization the kept softmax values are the gates.
    Margin follows [R&R] paragraph on the router margin: the k-th highest score
    minus the (k+1)-th highest; +inf when every expert is selected (k = N).
    """
    l = np.asarray(logits, np.float64)
    T, N = l.shape
    order = rank_experts(l)
    ids = order[:, :k]
    # READING: a NaN logit carries zero softmax weight (it already ranks last).
    lw = np.where(np.isnan(l), -np.inf, l)
    lmax = np.max(lw, axis=1, keepdims=True)
    with np.errstate(invalid="ignore", divide="ignore"):
        p = np.exp(lw - lmax)
        p = p / p.sum(axis=1, keepdims=True)        # softmax over all N experts
    sel = np.take_along_axis(p, ids, axis=1)
    with np.errstate(invalid="ignore", divide="ignore"):
        gates = sel / sel.sum(axis=1, keepdims=True) if renormalize else sel
    if k < N:
        lk = np.take_along_axis(l, order[:, k - 1:k + 1], axis=1)
        margin = lk[:, 0] - lk[:, 1]
    else:
        margin = np.full(T, np.inf)
    return ids.astype(np.int64), gates, margin


def replay_route(logits: np.ndarray, ids: np.ndarray, renormalize: bool = True):
    """Gates for recorded expert ids, and this run's router margin.

    [R&R] paragraph on router replay: the top-k expert indices of an earlier run are
    stored and used again, so the expert path of a later run is the same; it fixes the
    path only.  READING: only the indices are replayed; the gate weights come from
    this run's scores by the usual gate rule ([MIR] "How sparse routing works":
    softmax over all N, take the recorded experts, divide by their sum when
    renormalising).  An id outside [0, N) carries zero weight.  The margin is that of
    this run's own ranking ([R&R] margin paragraph), as topk_route gives it.

    Returns (gates [T, k] float64 in the recorded order, margin [T] float64).
    """
    l = np.asarray(logits, np.float64)
    ids = np.asarray(ids, np.int64)
    T, N = l.shape
    lw = np.where(np.isnan(l), -np.inf, l)
    lmax = np.max(lw, axis=1, keepdims=True)
    with np.errstate(invalid="ignore", divide="ignore"):
        p = np.exp(lw - lmax)
        p = p / p.sum(axis=1, keepdims=True)        # softmax over all N experts
    valid = (ids >= 0) & (ids < N)
    sel = np.where(valid, np.take_along_axis(p, np.clip(ids, 0, N - 1), axis=1), 0.0)
    with np.errstate(invalid="ignore", divide="ignore"):
        gates = sel / sel.sum(axis=1, keepdims=True) if renormalize else sel
    _, _, margin = topk_route(l, ids.shape[1], renormalize)
    return gates, margin


# ---------------------------------------------------------------- capacity and alignment

def capacity(T: int, k: int, N: int, cap_num: int, cap_den: int) -> Optional[int]:
    """Per-expert capacity, or None for dropless.

    [R&R] paragraph on expert capacity: tokens / experts x capacity factor.
    [MIR] "Worked example": capacity = int(mean per-expert load x factor), the mean
    load being T*k/N.  READING: both as floor(T*k*cap_num / (N*cap_den)) in
    integers, the factor given as the rational cap_num/cap_den; 0/0 = no limit.
    """
    if cap_num == 0 and cap_den == 0:
        return None
    return (T * k * cap_num) // (N * cap_den)


def capacity_keep(ids: np.ndarray, N: int, cap: Optional[int]) -> np.ndarray:
    """kept[r] for every route r = t*k + j (flattened ids).

    [R&R] paragraph on overflow: an expert over capacity overflows, the overflow
    skips the expert; a dispatcher that fills capacity in order makes batch
    position matter.  READING: capacity is filled in ascending route id, so a
    route is kept iff fewer than ``cap`` earlier routes went to its expert.
    Ids outside [0, N) are never kept.
    """
    flat = np.asarray(ids, np.int64).reshape(-1)
    kept = np.zeros(flat.shape[0], dtype=bool)
    used = [0] * N
    for r, e in enumerate(flat.tolist()):
        if not (0 <= e < N):
            continue
        if cap is None or used[e] < cap:
            kept[r] = True
            used[e] += 1
    return kept


def capacity_reroute(ids: np.ndarray, logits: np.ndarray, N: int, cap: Optional[int], depth: int):
    """Capacity with the reroute overflow policy.

    [MIR] "The hard part", Figure 2 (an expert at capacity: drop, or reroute -- send
    the token to its 2nd-choice expert) and the mitigation paragraph after the
    routing-stats probe (change the overflow policy from drop to reroute, sending
    overflow tokens to their second-choice expert).
    READING (rounds): first the drop policy fills capacity (capacity_keep).  Then up
    to ``depth`` rounds: in each, every token with an overflowed route offers its
    lowest such route one new candidate -- the next expert in the token's ranking of
    this run's logits (rank_experts) that is not among its recorded ids and was not
    offered before -- and requests are admitted in token order while the candidate
    has room left.  An admitted route runs the candidate with its original gate.
    depth 1 is the literal "second choice"; depth N - k walks the whole ranking.
    Routes with ids outside [0, N) never take part.

    Returns (expert [T*k] int64: the expert each route runs, -1 if none;
             kept [T*k] bool; rerouted [T*k] bool).
    """
    ids = np.asarray(ids, np.int64)
    T, k = ids.shape
    flat = ids.reshape(-1)
    kept = capacity_keep(ids, N, cap)
    expert = np.where(kept, flat, -1)
    rerouted = np.zeros(T * k, dtype=bool)
    if cap is None or depth <= 0:
        return expert, kept, rerouted
    room = [cap - int(np.count_nonzero(expert == e)) for e in range(N)]
    order = rank_experts(logits)
    cand = [[int(e) for e in order[t] if int(e) not in set(ids[t].tolist())] for t in range(T)]
    nxt = [0] * T
    for _ in range(depth):
        for t in range(T):
            pending = [j for j in range(k) if not kept[t * k + j] and 0 <= ids[t, j] < N]
            if not pending or nxt[t] >= len(cand[t]):
                continue
            c = cand[t][nxt[t]]
            nxt[t] += 1
            if room[c] > 0:
                r = t * k + pending[0]
                room[c] -= 1
                kept[r] = True
                expert[r] = c
                rerouted[r] = True
    return expert, kept, rerouted


def align(ids: np.ndarray, kept: np.ndarray, N: int, B: int):
    """Group kept routes by expert and pad each group to whole B-row blocks.

    [RB] "The bookkeeping before the matrix multiplication": routed rows are
    grouped by expert and padded into fixed-size blocks; route-block membership
    is the set of valid flattened route ids in each block.  [RB] "Stable
    construction selected a third trajectory": routes ordered by (expert id,
    flattened route id).  READING: flattened id r = t*k + j; each expert's list
    is padded to a multiple of B with the sentinel T*k; experts with no routes
    get no block; the buffers are sized for P_max = T*k + N*(B-1) rows.

    Returns dict with sorted_route_ids [P_max], block_expert [ceil(P_max/B)]
    (-1 past the end), expert_offsets [N+1], num_padded.
    """
    flat = np.asarray(ids, np.int64).reshape(-1)
    R = flat.shape[0]
    p_max = R + N * (B - 1)
    n_blocks = -(-p_max // B)
    sentinel = R
    sorted_ids = np.full(p_max, sentinel, dtype=np.int64)
    block_expert = np.full(n_blocks, -1, dtype=np.int64)
    offsets = np.zeros(N + 1, dtype=np.int64)
    pos = 0
    for e in range(N):
        members = np.nonzero(np.asarray(kept, bool) & (flat == e))[0]  # ascending route ids
        padded = -(-len(members) // B) * B
        sorted_ids[pos:pos + len(members)] = members
        block_expert[pos // B:(pos + padded) // B] = e
        pos += padded
        offsets[e + 1] = pos
    return {"sorted_route_ids": sorted_ids, "block_expert": block_expert,
            "expert_offsets": offsets, "num_padded": pos}


# ---------------------------------------------------------------- expert FFN and combine

def silu(x: np.ndarray) -> np.ndarray:
    """silu(x) = x / (1 + e^-x), written so that e^-x never overflows."""
    x = np.asarray(x, np.float64)
    out = np.empty_like(x)
    pos = x >= 0
    out[pos] = x[pos] / (1.0 + np.exp(-x[pos]))
    ex = np.exp(x[~pos])
    out[~pos] = x[~pos] * ex / (1.0 + ex)
    return out


def swiglu_expert(x: np.ndarray, w13: np.ndarray, w2: np.ndarray, stage_round=None) -> np.ndarray:
    """One SwiGLU expert on rows x [M, H]: y = W2 (silu(W1 x) * (W3 x)).

    w13 [2I, H]: rows 0..I-1 the gate projection W1, rows I..2I-1 the up
    projection W3 (the fused first projection "W13" of [RB] "The boundary that
    mattered"); w2 [H, I] the second projection.
    ``stage_round`` (diagnostic, default off) is applied to the weights, the
    activation and the output, to mimic a pipeline that stores them rounded.
    """
    r = stage_round if stage_round is not None else (lambda a: a)
    w13, w2 = r(w13), r(w2)
    I = w13.shape[0] // 2
    u = x @ w13[:I].T
    v = x @ w13[I:].T
    return r(r(silu(u) * v) @ w2.T)


def w13_projection(x: np.ndarray, w13: np.ndarray) -> np.ndarray:
    """The fused first projection on rows x [M, H]: [W1 x ; W3 x] -> [M, 2I].

    [RB] "The boundary that mattered" names the W13 output as the first of the four
    surfaces an expert row passes through.  Columns 0..I-1 are the gate projection
    (rows 0..I-1 of w13), columns I..2I-1 the up projection (rows I..2I-1).
    """
    return np.asarray(x, np.float64) @ np.asarray(w13, np.float64).T


def swiglu_activation(x: np.ndarray, w13: np.ndarray) -> np.ndarray:
    """The activation surface on rows x [M, H]: silu(W1 x) * (W3 x) -> [M, I].

    [RB] "The boundary that mattered": the activation is the surface between the W13
    output and the second projection; SwiGLU takes the gate half through silu and
    multiplies it by the up half.
    """
    u = w13_projection(x, w13)
    I = u.shape[1] // 2
    return silu(u[:, :I]) * u[:, I:]


def expert_ffn(h: np.ndarray, ids: np.ndarray, kept: np.ndarray, w13_of, w2_of, N: int,
               routes: Optional[np.ndarray] = None, stage_round=None) -> dict:
    """y_r = expert_{ids[r]}(h_{r // k}) for every kept route r (or the given subset).

    [MIR] "How sparse routing works": only the k selected experts run on a token.
    ``w13_of(e)`` / ``w2_of(e)`` return expert e's float64 weights.  Rows are
    grouped by expert only so that each expert's weights are materialised once;
    every row is computed independently.  Returns {route id: y row [H]}.
    """
    flat = np.asarray(ids, np.int64).reshape(-1)
    k = flat.shape[0] // h.shape[0]
    todo = np.nonzero(kept)[0] if routes is None else np.asarray([r for r in routes if kept[r]], np.int64)
    out = {}
    for e in range(N):
        rs = todo[flat[todo] == e]
        if rs.size == 0:
            continue
        y = swiglu_expert(np.asarray(h, np.float64)[rs // k], w13_of(e), w2_of(e), stage_round)
        for r, row in zip(rs.tolist(), y):
            out[r] = row
    return out


def combine(y_route: dict, gates: np.ndarray, kept: np.ndarray, T: int, H: int,
            shared: Optional[np.ndarray] = None, residual: Optional[np.ndarray] = None,
            tokens: Optional[np.ndarray] = None) -> np.ndarray:
    """out[t] = residual[t] + shared[t] + sum over kept j of gate[t, j] * y_{t*k+j}.

    [R&R] the simplified layer: output = sum of gate[e] * expert[e](h) over the
    chosen experts, fed back into the residual stream.  [MIR] "The hard part":
    a token whose route overflowed gets h plus only its surviving experts
    (Figure 2, drop branch).  READING: gates are not renormalised after a drop;
    absent terms are zero.  ``tokens`` restricts the rows computed.
    """
    g = np.asarray(gates, np.float64)
    k = g.shape[1]
    rows = np.arange(T) if tokens is None else np.asarray(tokens, np.int64)
    out = np.zeros((rows.shape[0], H), np.float64)
    for i, t in enumerate(rows.tolist()):
        acc = np.zeros(H, np.float64)
        for j in range(k):
            r = t * k + j
            if kept[r]:
                acc = acc + g[t, j] * y_route[r]
        if shared is not None:
            acc = acc + shared[i]
        if residual is not None:
            acc = acc + np.asarray(residual[t], np.float64)
        out[i] = acc
    return out


def routing_stats(ids: np.ndarray, kept: np.ndarray, N: int, cap: Optional[int]) -> dict:
    """Per-pass routing health numbers.

    [MIR] "Worked example": per-expert load is the bincount of the flattened top-k
    ids; overflow per expert is max(load - capacity, 0) and the dropped count is
    its sum.  [MIR] "The hard part": max/min load, imbalance = max / mean, drop
    fraction = dropped / total routed.
    """
    flat = np.asarray(ids, np.int64).reshape(-1)
    valid = (flat >= 0) & (flat < N)
    load = np.bincount(flat[valid], minlength=N)
    dropped = int(np.maximum(load - cap, 0).sum()) if cap is not None else 0
    total = int(load.sum())
    return {
        "load": load,
        "max_expert_load": int(load.max()),
        "min_expert_load": int(load.min()),
        "imbalance_ratio": float(load.max() / load.mean()) if total else 0.0,
        "dropped_tokens": dropped,
        "kept_routes": int(np.count_nonzero(kept)),
        "invalid_routes": int(np.count_nonzero(~valid)),
        "drop_fraction": dropped / total if total else 0.0,
        "capacity": -1 if cap is None else cap,
    }


def moe_forward(h, w_gate, w13_of, w2_of, *, k: int, B: int, cap_num: int = 0, cap_den: int = 0,
                renormalize: bool = True, bias=None, residual=None, shared_w13=None, shared_w2=None,
                logits=None, tokens=None, replay_ids=None, reroute_depth: int = 0) -> dict:
    """The whole layer, step after step in the pages' order, all in float64.

    route ([MIR] "How sparse routing works") -> capacity and drops ([R&R], [MIR]
    "The hard part") -> alignment ([RB]) -> expert FFN on kept routes -> combine.
    ``logits`` (if given) replaces the projection, for routing from stored logits.
    ``tokens`` restricts the expert FFN and combine to a sample of token rows.
    ``replay_ids`` (if given) are recorded expert ids used instead of this run's top-k
    ([R&R] router replay; gates from replay_route).  ``reroute_depth`` > 0 selects the
    reroute overflow policy (capacity_reroute) instead of dropping.
    """
    h = np.asarray(h, np.float64)
    T, H = h.shape
    N = (np.asarray(logits).shape[1] if logits is not None else np.asarray(w_gate).shape[0])
    l = router_logits(h, w_gate, bias) if logits is None else np.asarray(logits, np.float64)
    if replay_ids is None:
        ids, gates, margin = topk_route(l, k, renormalize)
    else:
        ids = np.asarray(replay_ids, np.int64).reshape(T, k)
        gates, margin = replay_route(l, ids, renormalize)
    cap = capacity(T, k, N, cap_num, cap_den)
    expert, kept, rerouted = capacity_reroute(ids, l, N, cap, reroute_depth)
    run_ids = np.where(kept.reshape(T, k), expert.reshape(T, k), ids)  # the expert each kept route runs
    al = align(run_ids, kept, N, B)
    rows = np.arange(T) if tokens is None else np.asarray(tokens, np.int64)
    routes = (rows[:, None] * k + np.arange(k)[None, :]).reshape(-1)
    y = expert_ffn(h, run_ids, kept, w13_of, w2_of, N, routes=routes)
    shared = None
    if shared_w13 is not None:
        shared = swiglu_expert(h[rows], shared_w13, shared_w2)
    out = combine(y, gates, kept, T, H, shared=shared, residual=residual, tokens=rows)
    stats = routing_stats(ids, kept, N, cap)
    stats["rerouted"] = int(np.count_nonzero(rerouted))
    stats["dropped_after_reroute"] = int(np.count_nonzero(~kept & (ids.reshape(-1) >= 0) & (ids.reshape(-1) < N)))
    return {"logits": l, "ids": ids, "gates": gates, "margin": margin, "cap": cap, "kept": kept,
            "run_ids": run_ids, "rerouted": rerouted, "align": al, "y_route": y, "shared": shared, "out": out,
            "tokens": rows, "stats": stats}


# ---------------------------------------------------------------- expert-choice routing
#
# [R&R] paragraph on expert-choice routing: the assignment is turned around, and each
# expert takes its highest-scoring tokens out of the whole batch.  [MIR] "Integration:
# where routing lives in a serving stack", paragraph on expert-choice routing (among the
# routing variants): each expert picks its tokens up to its capacity, so no expert
# overflows, and a token may be picked by no expert at all.

def expert_scores(logits: np.ndarray) -> np.ndarray:
    """Token-to-expert scores [T, N]: per token, the softmax over its N logits.

    READING: the score an expert ranks tokens by is the router's softmax probability
    ([MIR] "How sparse routing works" and the worked router: logits, then softmax over
    the experts).  A NaN logit weighs zero, as in topk_route.
    """
    l = np.asarray(logits, np.float64)
    lw = np.where(np.isnan(l), -np.inf, l)
    lmax = np.max(lw, axis=1, keepdims=True)
    with np.errstate(invalid="ignore", divide="ignore"):
        p = np.exp(lw - lmax)
        return p / p.sum(axis=1, keepdims=True)


def expert_choice_capacity(T: int, k: int, N: int, cap_num: int, cap_den: int) -> int:
    """Tokens each expert takes: C = min(floor(T*k*cf / N), T), cf = cap_num / cap_den.

    READING: the capacity formula of the token-choice layer ([R&R] capacity paragraph,
    [MIR] worked example), with k read as the average number of experts per token; an
    unset factor (0/0) means cf = 1, where expert choice runs as many expert rows as
    token-choice top-k.  An expert cannot take a token twice, so C <= T.
    """
    if cap_num == 0 and cap_den == 0:
        cap_num, cap_den = 1, 1
    return min((T * k * cap_num) // (N * cap_den), T)


def expert_choice_select(scores: np.ndarray, C: int):
    """Each expert's C highest-scoring tokens.

    Returns (tokens [N, C] int64: expert e's picks in ascending token order;
    slot [T, N] int64: position of token t in expert e's list, -1 if not picked;
    margin [N] float64: C-th highest score minus the (C+1)-th, +inf when C = 0 or C = T).
    READING: tokens are ranked by score descending, equal scores to the lower token
    index, a NaN score below every number (the token-choice tie rule applied to tokens).
    """
    S = np.asarray(scores, np.float64) + 0.0
    T, N = S.shape
    tokens = np.zeros((N, C), np.int64)
    slot = np.full((T, N), -1, np.int64)
    margin = np.full(N, np.inf)
    for e in range(N):
        # stable ascending sort of -score: highest first, equal scores in token order, NaN last
        order = np.argsort(-S[:, e], kind="stable")
        picked = np.sort(order[:C])
        tokens[e] = picked
        slot[picked, e] = np.arange(C)
        if 0 < C < T:
            margin[e] = S[order[C - 1], e] - S[order[C], e]
    return tokens, slot, margin


def expert_choice_align(tokens: np.ndarray, T: int, B: int) -> dict:
    """Expert e's picks as one segment of whole B-row blocks, experts in ascending order.

    Every expert has C picks, so segment e starts at e * Cp, Cp = ceil(C / B) * B, and
    holds the picked token ids ascending, then the sentinel T ([RB] "The bookkeeping
    before the matrix multiplication": expert-homogeneous padded blocks).
    """
    tokens = np.asarray(tokens, np.int64)
    N, C = tokens.shape
    Cp = -(-C // B) * B
    sorted_tokens = np.full(N * Cp, T, np.int64)
    for e in range(N):
        sorted_tokens[e * Cp:e * Cp + C] = tokens[e]
    return {"sorted_tokens": sorted_tokens, "block_expert": np.repeat(np.arange(N), Cp // B),
            "expert_offsets": np.arange(N + 1) * Cp, "num_padded": N * Cp, "segment": Cp}


def expert_choice_combine(y: dict, scores: np.ndarray, slot: np.ndarray, H: int,
                          shared: Optional[np.ndarray] = None, residual: Optional[np.ndarray] = None,
                          tokens: Optional[np.ndarray] = None) -> np.ndarray:
    """out[t] = residual[t] + shared[t] + sum over the experts e that picked t of score[t, e] * y_(t,e).

    READING: the gate of a pick is the token's score for that expert, not renormalised
    (a token's set of experts has no fixed size); a token no expert picked outputs its
    residual alone, like a fully dropped token ([MIR] "The hard part", drop branch).
    ``y`` maps (t, e) -> expert e's output row for token t.
    """
    S = np.asarray(scores, np.float64)
    T, N = S.shape
    rows = np.arange(T) if tokens is None else np.asarray(tokens, np.int64)
    out = np.zeros((rows.shape[0], H), np.float64)
    for i, t in enumerate(rows.tolist()):
        acc = np.zeros(H, np.float64)
        for e in range(N):
            if slot[t, e] >= 0:
                acc = acc + S[t, e] * y[(t, e)]
        if shared is not None:
            acc = acc + shared[i]
        if residual is not None:
            acc = acc + np.asarray(residual[t], np.float64)
        out[i] = acc
    return out


def expert_choice_forward(h, w_gate, w13_of, w2_of, *, k: int, B: int, cap_num: int = 0, cap_den: int = 0,
                          bias=None, residual=None, shared_w13=None, shared_w2=None, logits=None, scores=None,
                          tokens=None) -> dict:
    """The layer with expert-choice routing, all in float64.

    logits ([MIR] "How sparse routing works") -> scores -> each expert's top-C tokens
    -> padded segments -> SwiGLU expert FFN per pick -> score-weighted combine.
    ``logits`` / ``scores`` (if given) replace the projection / the softmax, for
    routing from stored values.  ``tokens`` restricts the FFN and combine to a sample.
    """
    h = np.asarray(h, np.float64)
    T, H = h.shape
    l = router_logits(h, w_gate, bias) if logits is None and scores is None else (
        None if logits is None else np.asarray(logits, np.float64))
    S = expert_scores(l) if scores is None else np.asarray(scores, np.float64)
    N = S.shape[1]
    C = expert_choice_capacity(T, k, N, cap_num, cap_den)
    picks, slot, margin = expert_choice_select(S, C)
    al = expert_choice_align(picks, T, B)
    rows = np.arange(T) if tokens is None else np.asarray(tokens, np.int64)
    y = {}
    for e in range(N):
        ts = [t for t in rows.tolist() if slot[t, e] >= 0]
        if ts:
            ye = swiglu_expert(h[ts], w13_of(e), w2_of(e))
            for t, row in zip(ts, ye):
                y[(t, e)] = row
    shared = swiglu_expert(h[rows], shared_w13, shared_w2) if shared_w13 is not None else None
    out = expert_choice_combine(y, S, slot, H, shared=shared, residual=residual, tokens=rows)
    picks_per_token = np.count_nonzero(slot >= 0, axis=1)
    stats = {"capacity": C, "picks": N * C, "unpicked_tokens": int(np.count_nonzero(picks_per_token == 0)),
             "max_picks": int(picks_per_token.max()) if T else 0}
    return {"logits": l, "scores": S, "cap": C, "tokens": picks, "slot": slot, "margin": margin, "align": al,
            "y": y, "shared": shared, "out": out, "rows": rows, "stats": stats}
