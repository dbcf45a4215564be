/*
 * moe.h -- C ABI of libmoe_mi355x.so: the Mixture-of-Experts layer forward pass on
 * AMD Instinct MI355X (gfx950), with token-choice routing (below) or expert-choice
 * routing (moe_route_expert_choice and its companions, further down).
 *
 * Per token the layer computes (pages cited by title and section):
 *   1. router logits  l = h . W_g^T (+ optional per-expert bias)
 *        "Mixture-of-Experts Routing at Inference Time", "How sparse routing works"
 *        and "Worked example: a top-k router and the imbalance it produces";
 *   2. top-k experts by (logit descending, lower expert index on ties), softmax
 *      gates renormalised over the k chosen, and the router margin (k-th minus
 *      (k+1)-th logit)
 *        same page and section; "Mixture-of-experts routing & LLM repeatability",
 *        paragraphs on the top-k step and on the router margin;
 *   3. an optional per-expert capacity, filled in route order, whose overflow
 *      routes are dropped to the residual path
 *        "Mixture-of-experts routing & LLM repeatability", paragraph on expert
 *        capacity; "Mixture-of-Experts Routing at Inference Time", "The hard part:
 *        token dropping is a silent correctness bug", Figure 2;
 *   4. alignment of kept routes into expert-homogeneous blocks of B rows, ordered
 *      by (expert id, flattened route id), padded with a sentinel
 *        "Route-Block Membership Selects Packed-AWQ Arithmetic", sections "The
 *        bookkeeping before the matrix multiplication" and "Stable construction
 *        selected a third trajectory";
 *   5. SwiGLU expert FFNs on the aligned rows: fused first projection W13
 *      (gate rows, then up rows), silu(gate) * up, second projection W2
 *        same page, "The boundary that mattered" (W13, activation, W2 surfaces);
 *   6. gate-weighted combine added to the residual stream
 *        "Mixture-of-Experts Routing at Inference Time", "How sparse routing
 *        works" and Figure 2.
 *
 * Conventions for every entry point
 *   - Tensors are dense, row-major, and live in device memory (pointers from
 *     hipMalloc or a torch CUDA tensor).  Data tensors (h, weights, act, y, out,
 *     residual, logits) must be 16-byte aligned; int32/float32 index and gate
 *     arrays 4-byte aligned; byte arrays unaligned.
 *   - The caller owns and allocates every buffer, including the workspace whose
 *     size moe_workspace_size reports.  The library allocates nothing, keeps no
 *     pointer after return and has no global state besides its code object.
 *   - `stream` is a hipStream_t (NULL = the null stream).  All work is enqueued
 *     asynchronously on it; buffers must stay alive until it completes.
 *   - Arguments are validated on the host first.  On any error nothing is
 *     enqueued and an error code is returned; no exception crosses the ABI.
 *     A failed kernel launch returns MOE_ERR_HIP.
 *   - Route id r = t*k + j for token t and rank j (0 = highest).  The padding
 *     sentinel is T*k.  P_max = T*k + N*(B-1) bounds the padded row count.
 *   - Every reduction has a fixed split and order that depends only on the
 *     config (never on T or on other tokens), so each token's logits, ids,
 *     gates, expert outputs and layer output are bitwise identical whatever
 *     else is in the batch (dropless configs; with a capacity limit the drop
 *     decisions themselves depend on the batch, as the pages say).
 */
#ifndef MOE_MI355X_H_
#define MOE_MI355X_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 5

typedef int32_t moe_status;
enum {
  MOE_OK = 0,
  MOE_ERR_NULL_POINTER = 1,        /* a required pointer is NULL */
  MOE_ERR_INVALID_CONFIG = 2,      /* config outside the supported envelope */
  MOE_ERR_UNSUPPORTED = 3,         /* dtype combination or flag not implemented */
  MOE_ERR_MISALIGNED = 4,          /* pointer alignment rule violated */
  MOE_ERR_WORKSPACE_TOO_SMALL = 5, /* ws_bytes below moe_workspace_size */
  MOE_ERR_HIP = 6                  /* a HIP runtime call or kernel launch failed */
};

/* Element types.  fp8 is OCP E4M3FN (bias 7, max 448, no infinities). */
enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_FP8_E4M3 = 2 };

/* moe_route flags (may be combined) */
enum {
  MOE_ROUTE_LOGITS_IN = 1u, /* skip the projection: `logits` is an input (stored or replayed logits) */
  MOE_ROUTE_IDS_IN = 2u,    /* router replay: `topk_ids` is an input (recorded expert ids) */
  MOE_ROUTE_NO_LOGITS_OUT = 4u /* the logits are not written (`logits` may be NULL); bf16
                                  activations only, not with MOE_ROUTE_LOGITS_IN */
};

/* moe_config.routing */
enum {
  MOE_ROUTING_TOKEN_CHOICE = 0, /* each token picks its top-k experts */
  MOE_ROUTING_EXPERT_CHOICE = 1 /* each expert picks its top-C tokens */
};

/* moe_workspace_size operations */
enum { MOE_OP_ALIGN = 1, MOE_OP_FORWARD = 2 };

/* Offsets into the stats array written by moe_align ([N + MOE_STATS_EXTRA] int32). */
enum {
  MOE_STAT_KEPT = 0,      /* routes kept (stats[N + 0]) */
  MOE_STAT_DROPPED = 1,   /* valid routes dropped by capacity */
  MOE_STAT_INVALID = 2,   /* routes whose expert id is outside [0, N) (never kept) */
  MOE_STAT_CAPACITY = 3,  /* per-expert capacity, -1 when dropless */
  MOE_STAT_MAX_LOAD = 4,  /* max over experts of routed load (before capacity) */
  MOE_STAT_MIN_LOAD = 5,  /* min over experts of routed load */
  MOE_STAT_NUM_PADDED = 6,/* padded rows used (same as *num_padded) */
  MOE_STAT_REROUTED = 7,  /* routes kept by rerouting to another expert (reroute policy) */
  MOE_STAT_UNPICKED = 8,  /* expert choice: tokens that no expert picked (0 for token choice) */
  MOE_STAT_MAX_PICKS = 9, /* expert choice: most experts that picked one token (0 for token choice) */
  MOE_STATS_EXTRA = 10
};

/*
 * Layer shape and numerics.  Supported envelope:
 *   1 <= T <= 65536;  H, I multiples of 128, 128 <= H, I <= 32768;
 *   1 <= N <= 256;  1 <= k <= min(8, N);  B in {8, 16, 32, 64, 128};
 *   capacity factor cap_num/cap_den > 0, or 0/0 for dropless:
 *     cap = floor(T*k*cap_num / (N*cap_den))  (may be 0: every route dropped);
 *   n_shared in {0, 1} (one always-on expert added with gate 1);
 *   renormalize 1 = gates renormalised over the k chosen, 0 = plain softmax values;
 *   dtypes: (act F32, expert F32), (act BF16, expert BF16),
 *           (act BF16, expert FP8_E4M3 with scale_block 128);
 *   bf16 activations: T*H < 2^31 and 2*I*H < 2^31 (the expert GEMMs address h
 *           and one expert's weights with 32-bit byte offsets);
 *   0 <= reroute_depth <= N - k: overflow policy under capacity.  0 = drop ("Mixture-
 *           of-Experts Routing at Inference Time", "The hard part", Figure 2, drop
 *           branch); d > 0 = reroute (Figure 2's reroute branch, and the mitigation
 *           paragraph after the routing-stats probe): after the drop-policy fill, up to
 *           d rounds in which each token with an overflowed route offers its lowest such
 *           route the next expert of its own ranking not among its ids and not offered
 *           before; requests are admitted in token order while the expert has room.  The
 *           route keeps its gate.  d = 1 is the "second choice"; see moe_align_reroute.
 *   routing: MOE_ROUTING_TOKEN_CHOICE, or MOE_ROUTING_EXPERT_CHOICE (needs
 *           reroute_depth 0; see moe_route_expert_choice for what k and the capacity
 *           factor mean there, and which entry points apply).
 * act_dtype is the type of h, residual, out, W_g, act and y_route.
 */
typedef struct moe_config {
  uint32_t struct_size; /* sizeof(moe_config) */
  int32_t T, H, N, k, I, B;
  int32_t cap_num, cap_den;
  int32_t n_shared;
  int32_t renormalize;
  int32_t act_dtype;
  int32_t expert_dtype;
  int32_t scale_block;  /* 128 for fp8 experts, else 0 */
  int32_t reroute_depth; /* 0 = drop overflow; > 0 = reroute rounds (see above) */
  int32_t routing;       /* MOE_ROUTING_TOKEN_CHOICE or MOE_ROUTING_EXPERT_CHOICE */
} moe_config;

/*
 * Weights for moe_forward / moe_expert_ffn (device pointers).
 *   w_gate      [N, H] act dtype (router projection, one row per expert)
 *   logit_bias  [N] float32, nullable (added to the logits)
 *   w13         [N, 2I, H] expert dtype: rows 0..I-1 gate projection, I..2I-1 up projection
 *   w2          [N, H, I] expert dtype
 *   w13_scale   fp8 only: [N, 2I/128, H/128] bf16, w = e4m3(q) * scale of its 128x128 block
 *   w2_scale    fp8 only: [N, H/128, I/128] bf16
 *   shared_*    the always-on expert, same layouts without the N dimension (n_shared = 1)
 */
typedef struct moe_weights {
  const void* w_gate;
  const float* logit_bias;
  const void* w13;
  const void* w2;
  const void* w13_scale;
  const void* w2_scale;
  const void* shared_w13;
  const void* shared_w2;
  const void* shared_w13_scale;
  const void* shared_w2_scale;
} moe_weights;

/*
 * Optional places for moe_forward's intermediates.  Any non-NULL member is
 * used instead of the workspace region for that tensor, so the caller can read
 * it after the stream completes (route traces, replay, debugging).
 */
typedef struct moe_trace {
  float* logits;             /* [T, N] */
  /* token choice */
  int32_t* topk_ids;         /* [T, k] */
  float* topk_gates;         /* [T, k] */
  float* margin;             /* [T] */
  uint8_t* route_kept;       /* [T*k] */
  int32_t* sorted_route_ids; /* [P_max] */
  int32_t* block_expert;     /* [ceil(P_max / B)] */
  int32_t* expert_offsets;   /* [N + 1] */
  int32_t* num_padded;       /* [1] */
  int32_t* stats;            /* [N + MOE_STATS_EXTRA] */
  void* act;                 /* [P_max, I] act dtype */
  void* y_route;             /* [T*k, H] act dtype */
  int32_t* route_expert;     /* [T*k]: expert each route runs, -1 none (reroute policy only) */
  /* expert choice (sorted_route_ids then holds token ids, y_route is [P, H] by padded row) */
  float* scores;             /* [T, N] */
  int32_t* choice_tokens;    /* [N, C] */
  int32_t* choice_slot;      /* [T, N] */
  float* choice_margin;      /* [N] */
  /* Nullable: MOE_TRACE_EVENTS HIP events (hipEvent_t, created by the caller, with timing
   * enabled), recorded on the forward's stream around its stages: [0] before the router,
   * [1] after routing (expert choice: scores and picks), [2] after the alignment, [3]
   * after the W13 + SwiGLU GEMM, [4] after the W2 GEMM, [5] after the shared expert (the
   * same point as [4] without one), [6] after the combine.  The time between two
   * consecutive events is that stage as it runs inside the layer.  A failed record is
   * returned as MOE_ERR_HIP. */
  void* const* stage_events;
  /* Nullable: [P_max, 2I] act dtype, the routed W13 output before the activation (columns
   * 0..I-1 the gate projection, I..2I-1 the up projection; see moe_expert_gate_up). */
  void* w13_out;
  /* Nullable, 8-byte aligned: [2][MOE_CLOCK_SLOTS][4] uint64, clock stamps of the routed W13
   * ([0]) and W2 ([1]) GEMM launches.  Persistent workgroup b writes, at its start, the
   * core-cycle counter (HIP clock64) and the constant-rate wall-clock counter (HIP
   * wall_clock64, rate hipDeviceAttributeWallClockRate) into [.][b][0..1], and both again at
   * its end into [.][b][2..3]: (t_end - t_start) / (r_end - r_start) times the wall-clock
   * rate is the clock that workgroup ran at.  Slots of workgroups a launch does not have are
   * not written. */
  uint64_t* gemm_clocks;
} moe_trace;

#define MOE_CLOCK_SLOTS 1024

#define MOE_TRACE_EVENTS 7

/* ABI version (MOE_ABI_VERSION) of the loaded library. */
int32_t moe_abi_version(void);

/* Static text for a status code; never NULL. */
const char* moe_status_str(moe_status s);

/* Host-only check of a config against the supported envelope. */
moe_status moe_validate_config(const moe_config* cfg);

/* Host-only: the padded row bound P and ceil(P / B) for a valid config: token choice
 * P = P_max = T*k + N*(B-1); expert choice P = N * ceil(C / B) * B (exact). */
moe_status moe_align_sizes(const moe_config* cfg, int32_t* p_max, int32_t* n_blocks);

/* Host-only: workspace bytes needed by moe_align (MOE_OP_ALIGN) or moe_forward (MOE_OP_FORWARD). */
moe_status moe_workspace_size(const moe_config* cfg, int32_t op, size_t* bytes);

/*
 * Router: projection, top-k, gates, margin.
 *   h          [T, H] act dtype (ignored with MOE_ROUTE_LOGITS_IN)
 *   w_gate     [N, H] act dtype (ignored with MOE_ROUTE_LOGITS_IN)
 *   logit_bias [N] float32, nullable (ignored with MOE_ROUTE_LOGITS_IN)
 *   logits     [T, N] float32: written, or read with MOE_ROUTE_LOGITS_IN; with
 *              MOE_ROUTE_NO_LOGITS_OUT nullable and not written (bf16 activations: the
 *              logits stay on chip between the projection and the top-k)
 *   topk_ids   [T, k] int32, rank order;  topk_gates [T, k] float32
 *   margin     [T] float32, nullable: l_(k-1) - l_(k) in rank order, +inf when k = N
 * Logits are accumulated in fp32 over fixed 32-wide K steps in ascending K.
 * A NaN logit ranks below every number and carries zero gate weight; -0 == +0.
 *
 * MOE_ROUTE_IDS_IN, router replay ("Mixture-of-experts routing & LLM repeatability",
 * router replay paragraph: the top-k indices of an earlier run are stored and used
 * again, fixing the expert path): topk_ids holds recorded expert ids and is only
 * read.  topk_gates are then this run's gates over those experts in their recorded
 * order: exp(l_id - m) / sum over the recorded ids (m their largest logit), or the
 * plain softmax values with renormalize = 0; an id outside [0, N) weighs 0 (a token
 * with no valid id gets NaN gates, 0/0, and moe_align never keeps its routes).  The
 * margin is this run's own (how close its scores are to a different route).
 * Replaying a run's own ids reproduces its gates bit for bit.
 */
moe_status moe_route(const moe_config* cfg, const void* h, const void* w_gate, const float* logit_bias,
                     float* logits, int32_t* topk_ids, float* topk_gates, float* margin, uint32_t flags,
                     void* stream);

/*
 * Capacity with the drop policy (whatever reroute_depth says; moe_align_reroute
 * applies the config's policy) and alignment (deterministic: no atomic decides any order).
 *   capacity: "Mixture-of-experts routing & LLM repeatability", paragraph on expert
 *     capacity (tokens / experts x factor, filled in batch order, overflow skips the
 *     expert); "Mixture-of-Experts Routing at Inference Time", "Worked example" (the
 *     capacity as the mean load times the factor, drops = overflow summed over experts)
 *     and "The hard part", Figure 2 (drop branch: the token keeps only the residual path);
 *   alignment: "Route-Block Membership Selects Packed-AWQ Arithmetic", "The bookkeeping
 *     before the matrix multiplication" (rows grouped by expert, padded into fixed-size
 *     blocks; membership = the valid flattened route ids of a block) and "Stable
 *     construction selected a third trajectory" (order by expert id, then route id);
 *   stats: "Mixture-of-Experts Routing at Inference Time", "Worked example" (per-expert
 *     load = bincount of the flattened ids) and "The hard part" (the routing-stats probe).
 *   topk_ids         [T*k] int32 (from moe_route, or replayed by the caller)
 *   route_kept       [T*k] uint8 out: 1 = the route runs its expert, 0 = dropped or invalid id
 *   sorted_route_ids [P_max] int32 out: per expert (ascending), its kept route ids ascending,
 *                    padded to a multiple of B with the sentinel T*k; the tail is sentinel
 *   block_expert     [ceil(P_max/B)] int32 out: expert of each B-row block, -1 past the end
 *   expert_offsets   [N+1] int32 out: first padded row of each expert; [N] = padded rows used
 *   num_padded       [1] int32 out
 *   stats            [N + MOE_STATS_EXTRA] int32 out, nullable: per-expert load, then the
 *                    MOE_STAT_* counters
 *   ws, ws_bytes     device workspace of at least moe_workspace_size(MOE_OP_ALIGN) bytes
 */
moe_status moe_align(const moe_config* cfg, const int32_t* topk_ids, uint8_t* route_kept,
                     int32_t* sorted_route_ids, int32_t* block_expert, int32_t* expert_offsets,
                     int32_t* num_padded, int32_t* stats, void* ws, size_t ws_bytes, void* stream);

/*
 * Capacity with the config's overflow policy (reroute when reroute_depth > 0), then
 * the alignment of the routes as they run.  Arguments as moe_align, plus:
 *   logits       [T, N] float32: this run's scores; each token's candidates are its
 *                experts in ranking order (value descending, lower index first, NaN
 *                last, -0 == +0) without its topk_ids
 *   route_expert [T*k] int32 out: the expert each route runs (its own id, the expert
 *                it was rerouted to, or -1 when dropped or invalid)
 * sorted_route_ids, block_expert and expert_offsets group the routes by route_expert;
 * stats[N + MOE_STAT_REROUTED] counts routes kept by rerouting, DROPPED those left
 * without an expert; per-expert loads are before capacity.  The decisions are made by
 * one workgroup in token order (no atomic decides an order).  With reroute_depth 0
 * the result equals moe_align's (plus route_expert).
 */
moe_status moe_align_reroute(const moe_config* cfg, const int32_t* topk_ids, const float* logits,
                             int32_t* route_expert, uint8_t* route_kept, int32_t* sorted_route_ids,
                             int32_t* block_expert, int32_t* expert_offsets, int32_t* num_padded, int32_t* stats,
                             void* ws, size_t ws_bytes, void* stream);

/*
 * Grouped SwiGLU expert FFN over aligned rows ("Route-Block Membership Selects
 * Packed-AWQ Arithmetic", "The boundary that mattered": an expert row passes through the
 * fused first projection W13, the activation and the routed second projection W2; the
 * page compares exactly these surfaces).  The FFN form is SwiGLU, the gate half through
 * silu times the up half ("Mixture-of-Experts Routing at Inference Time", "How sparse
 * routing works": each chosen expert is a feed-forward network applied to h).
 * Routed mode (sorted_route_ids != NULL): rows p in expert e's segment
 *   [expert_offsets[e], expert_offsets[e+1]) hold route r = sorted_route_ids[p]
 *   (token r / k); sentinel rows compute zeros and write no output row.
 *   w13/w2 (+ scales) are the [N, ...] stacks; act is [P_max, I]; y_out is
 *   y_route [T*k, H]: row r written for every kept route, other rows untouched.
 * Identity mode (sorted_route_ids == NULL, expert_offsets ignored): one expert
 *   (w13 [2I, H], w2 [H, I]) on every token row t; act is [T, I]; y_out is [T, H].
 * act = silu(h W1^T) * (h W3^T) is stored in the act dtype (fp32 accumulation);
 * fp8 weights are decoded and scaled to bf16 before the bf16 MFMA.  Every row's
 * K order is fixed, so a row's results do not depend on the other rows.
 *   w13_out  nullable debug surface [P_max, 2I] (identity mode [T, 2I]), act dtype: the W13
 *            output before the activation, columns 0..I-1 = h W1^T, I..2I-1 = h W3^T, each
 *            rounded once from its fp32 accumulator (the same accumulators act is made
 *            from); rows as act.  Leaves act and y_out bit for bit unchanged.
 */
moe_status moe_expert_ffn(const moe_config* cfg, const void* h, const int32_t* sorted_route_ids,
                          const int32_t* expert_offsets, const void* w13, const void* w2,
                          const void* w13_scale, const void* w2_scale, void* act, void* w13_out,
                          void* y_out, void* stream);

/*
 * The two halves of moe_expert_ffn, for callers that want the surfaces apart
 * (same row conventions and modes as moe_expert_ffn):
 *   moe_expert_gate_up: act = silu(x W1^T) * (x W3^T) from the fused W13 projection
 *                       ("Route-Block Membership Selects Packed-AWQ Arithmetic", "The
 *                       boundary that mattered": W13 and activation surfaces); w13_out
 *                       (nullable) as moe_expert_ffn's;
 *   moe_expert_down:    y rows = act W2^T (the routed second projection surface).
 */
moe_status moe_expert_gate_up(const moe_config* cfg, const void* h, const int32_t* sorted_route_ids,
                              const int32_t* expert_offsets, const void* w13, const void* w13_scale, void* act,
                              void* w13_out, void* stream);
moe_status moe_expert_down(const moe_config* cfg, const void* act, const int32_t* sorted_route_ids,
                           const int32_t* expert_offsets, const void* w2, const void* w2_scale, void* y_out,
                           void* stream);

/*
 * Combine ("Mixture-of-experts routing & LLM repeatability", the layer sketch: the output
 * is the gate-weighted sum of the chosen experts' outputs, fed back into the residual
 * stream; "Mixture-of-Experts Routing at Inference Time", "How sparse routing works",
 * Figure 1, and "The hard part", Figure 2: a dropped route contributes nothing, the token
 * keeps h and its surviving experts; "When Faster ≠ Identical: Numerical Pitfalls in
 * Serving MoE Models", "Why This Matters": the always-on shared expert is added to the
 * routed output):
 *   out[t] = round( ((sum over kept j ascending of gate[t,j] * y_route[t*k+j])
 *                    + shared_out[t]) + residual[t] ), fp32 accumulation in exactly
 * that order, one rounding to the act dtype.  Gates are not renormalised after a drop.
 * A token with no kept route, no shared expert and a residual outputs its residual bitwise.
 *   y_route [T*k, H], topk_gates [T, k] float32, route_kept [T*k] uint8,
 *   shared_out [T, H] nullable, residual [T, H] nullable, out [T, H]; all act dtype but gates.
 */
moe_status moe_combine(const moe_config* cfg, const void* y_route, const float* topk_gates,
                       const uint8_t* route_kept, const void* shared_out, const void* residual,
                       void* out, void* stream);

/*
 * The whole layer ("Mixture-of-Experts Routing at Inference Time", "How sparse routing
 * works", Figure 1: router, top-k, the chosen experts, weighted sum; "Mixture-of-experts
 * routing & LLM repeatability", the layer sketch), as the entry points above compose it:
 * moe_route -> moe_align -> moe_expert_ffn (routed, then the shared
 * expert in identity mode) -> moe_combine, on one stream, with no host synchronisation.
 *   h [T, H], residual [T, H] nullable (pass h for the usual h + MoE(h)), out [T, H].
 *   trace nullable (see moe_trace); ws of moe_workspace_size(MOE_OP_FORWARD) bytes.
 */
moe_status moe_forward(const moe_config* cfg, const moe_weights* weights, const void* h,
                       const void* residual, void* out, const moe_trace* trace, void* ws,
                       size_t ws_bytes, void* stream);

/*
 * moe_forward without a workspace, for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * composition, kernels and results bit for bit, with every intermediate in a static scratch
 * array of MOE_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs on until the
 * process ends.  The caller still passes inputs, outputs and (nullable) trace buffers.
 *   Limit: configs whose forward workspace (moe_workspace_size, MOE_OP_FORWARD) exceeds
 *   MOE_NOALLOC_SCRATCH_BYTES return MOE_ERR_WORKSPACE_TOO_SMALL and enqueue nothing (it
 *   holds, e.g., a Mixtral-shaped layer (H 4096, 8 experts, top-2, I 14336, B 64) up to 1622
 *   tokens, a Qwen3-MoE-shaped one up to 2871, a DeepSeek-V3-shaped one up to 407).
 *   The scratch is that of the current device (hipGetDevice); `stream` must belong to it.
 *   Calls on one GPU share its scratch: calls that overlap on the GPU (on different streams,
 *   or from different host threads without ordering) race.  Calls in one stream order are safe.
 *   The first call on a device looks up the scratch's device address; no call allocates.
 *   A failed lookup returns MOE_ERR_HIP.
 */
#define MOE_NOALLOC_SCRATCH_BYTES (128u << 20)
moe_status moe_forward_noalloc(const moe_config* cfg, const moe_weights* weights, const void* h,
                               const void* residual, void* out, const moe_trace* trace, void* stream);

/*
 * The whole layer with router replay ("Mixture-of-experts routing & LLM
 * repeatability", router replay paragraph): as moe_forward, but the experts are the
 * recorded ids instead of this run's top-k (moe_route with MOE_ROUTE_IDS_IN);
 * capacity, alignment, expert FFN and combine run on them.
 *   replay_ids [T, k] int32, recorded expert ids (e.g. trace->topk_ids of an earlier
 *              moe_forward); only read.  trace->topk_ids is not used.
 * Everything else as moe_forward, same workspace size.  Replaying a run's own ids
 * reproduces its output bit for bit.  Returns MOE_ERR_NULL_POINTER for a NULL
 * replay_ids and MOE_ERR_MISALIGNED if it is not 4-byte aligned.
 */
moe_status moe_forward_replay(const moe_config* cfg, const moe_weights* weights, const void* h,
                              const void* residual, const int32_t* replay_ids, void* out,
                              const moe_trace* trace, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------- expert-choice routing
 *
 * "Mixture-of-experts routing & LLM repeatability", paragraph on expert-choice routing:
 * the assignment is turned around, and each expert takes its highest-scoring tokens from
 * the whole batch.  "Mixture-of-Experts Routing at Inference Time", "Integration: where
 * routing lives in a serving stack", paragraph on expert-choice routing: each expert picks
 * up to its capacity, so no expert overflows, and a token may be picked by no expert.
 *
 * For a config with routing = MOE_ROUTING_EXPERT_CHOICE:
 *   score[t, e]  = softmax over the N logits of token t (the router's probabilities; a
 *                  NaN logit weighs 0).  For a token's top-k experts these are bitwise the
 *                  token-choice gates with renormalize = 0.
 *   C            = min(floor(T*k*cap_num / (N*cap_den)), T) tokens per expert, the factor
 *                  being 1 when cap_num = cap_den = 0 (k reads as the mean number of
 *                  experts per token; factor 1 runs as many expert rows as top-k).
 *   picks        expert e takes the C tokens ranked first by (score descending, lower token
 *                index first, NaN last).
 *   gate         a pick's gate is its score, not renormalised.  out[t] = round(((sum over
 *                the experts that picked t, ascending e, of score[t,e] * y) + shared[t])
 *                + residual[t]); a token no expert picked outputs its residual bitwise.
 *   rows         P = N * Cp padded rows, Cp = ceil(C / B) * B: expert e's picks at rows
 *                [e*Cp, e*Cp + C) in ascending token order, sentinel T after them.
 * Entry points: moe_route_expert_choice, moe_align_expert_choice, moe_expert_ffn /
 * moe_expert_gate_up / moe_expert_down (sorted_route_ids then holds token ids with the
 * sentinel T, and y_out is [P, H], written at each real padded row), moe_combine_expert_choice
 * and moe_forward (trace: logits, scores, choice_*, sorted_route_ids, block_expert,
 * expert_offsets, num_padded, stats, act, y_route).  moe_route, moe_align,
 * moe_align_reroute, moe_combine and moe_forward_replay return MOE_ERR_UNSUPPORTED for such
 * a config, and the expert-choice entry points do for a token-choice config.  The picks
 * depend on the whole batch by construction: no batch invariance is claimed, only that the
 * same inputs give the same bits.
 */

/* Host-only, expert-choice config: C (tokens per expert) and Cp = ceil(C / B) * B. */
moe_status moe_expert_choice_sizes(const moe_config* cfg, int32_t* capacity, int32_t* segment);

/*
 * Scores and each expert's picks.
 *   h, w_gate, logit_bias, logits: as moe_route (MOE_ROUTE_LOGITS_IN: logits are read)
 *   scores        [T, N] float32 out
 *   choice_tokens [N, C] int32 out: expert e's picks, ascending token ids (nothing if C = 0)
 *   choice_slot   [T, N] int32 out: position of t in expert e's list, -1 if not picked
 *   choice_margin [N] float32 out, nullable: C-th minus (C+1)-th highest score of expert e
 *                 (0 on a tie at the cut), +inf when C = 0 or C = T
 * One workgroup per expert selects with a radix select over the 32-bit score keys (counts
 * only, no atomic decides an order) and lists its picks with prefix counts in token order.
 * Flags other than MOE_ROUTE_LOGITS_IN return MOE_ERR_UNSUPPORTED.
 */
moe_status moe_route_expert_choice(const moe_config* cfg, const void* h, const void* w_gate,
                                   const float* logit_bias, float* logits, float* scores,
                                   int32_t* choice_tokens, int32_t* choice_slot, float* choice_margin,
                                   uint32_t flags, void* stream);

/*
 * Padded rows of the picks (no workspace).
 *   choice_tokens, choice_slot   from moe_route_expert_choice
 *   sorted_route_ids [P] int32 out: token ids per expert segment, sentinel T as padding
 *   block_expert     [P / B] int32 out;  expert_offsets [N+1] int32 out (e * Cp);
 *   num_padded       [1] int32 out (P)
 *   stats            [N + MOE_STATS_EXTRA] int32 out, nullable: C per expert, KEPT = N*C,
 *                    CAPACITY = C, MAX_LOAD = MIN_LOAD = C, NUM_PADDED = P, UNPICKED and
 *                    MAX_PICKS from choice_slot, the others 0
 */
moe_status moe_align_expert_choice(const moe_config* cfg, const int32_t* choice_tokens,
                                   const int32_t* choice_slot, int32_t* sorted_route_ids,
                                   int32_t* block_expert, int32_t* expert_offsets, int32_t* num_padded,
                                   int32_t* stats, void* stream);

/*
 * Combine of the picks: out[t] = round(((sum over e ascending with choice_slot[t,e] >= 0 of
 * scores[t,e] * y_rows[e*Cp + choice_slot[t,e]]) + shared_out[t]) + residual[t]), fp32,
 * one rounding.  y_rows [P, H], scores and choice_slot [T, N], shared_out / residual
 * nullable [T, H], out [T, H]; act dtype but scores and slots.
 */
moe_status moe_combine_expert_choice(const moe_config* cfg, const void* y_rows, const float* scores,
                                     const int32_t* choice_slot, const void* shared_out, const void* residual,
                                     void* out, void* stream);

/* ---------------------------------------------------------------- routing health
 *
 * "Mixture-of-Experts Routing at Inference Time", "Worked example" (per-expert load and the
 * dropped count) and "The hard part" (the per-pass routing-stats probe: largest and smallest
 * expert load, imbalance = largest load over the mean load, dropped routes and their share
 * of all routed ones, exported as a metric every forward pass).
 */
typedef struct moe_routing_health {
  int32_t total_routes;     /* routes with an expert id in [0, N): the sum of the per-expert loads */
  int32_t max_expert_load;  /* per-expert load before capacity */
  int32_t min_expert_load;
  int32_t dropped_routes;   /* valid routes that run no expert (MOE_STAT_DROPPED) */
  int32_t kept_routes;      /* routes that run an expert (MOE_STAT_KEPT) */
  int32_t invalid_routes;   /* ids outside [0, N) (MOE_STAT_INVALID) */
  int32_t capacity;         /* per-expert capacity, -1 when dropless */
  int32_t rerouted_routes;  /* reroute policy: kept on another expert (MOE_STAT_REROUTED) */
  int32_t unpicked_tokens;  /* expert choice: tokens no expert picked (MOE_STAT_UNPICKED) */
  int32_t reserved;         /* 0 */
  double imbalance_ratio;   /* max_expert_load / (total_routes / N); 0 when total_routes = 0 */
  double drop_fraction;     /* dropped_routes / total_routes; 0 when total_routes = 0 */
} moe_routing_health;

/* Host-only: the routing-health numbers of one pass from the stats array that moe_align,
 * moe_align_reroute, moe_align_expert_choice or moe_forward (trace->stats) wrote, after the
 * caller has copied it to host memory ([N + MOE_STATS_EXTRA] int32).  Reads nothing on the
 * device and enqueues nothing.  MOE_ERR_NULL_POINTER for a NULL stats or out;
 * MOE_ERR_INVALID_CONFIG for an invalid config, or a stats array that no alignment of this
 * config can have written (a negative load or counter). */
moe_status moe_routing_health_from_stats(const moe_config* cfg, const int32_t* stats, moe_routing_health* out);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H_ */
