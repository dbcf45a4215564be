// Internal launch entry points between the host layer (api.hip) and the kernels.
// Every launcher enqueues on `stream` and returns hipSuccess or the launch error.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

// ---- routing (route.hip)
// projection + top-k + gates + margin (fused for bf16).  replay (nullable): recorded
// expert ids [T, k]; gates are then taken over them and ids is not written.
// scores (nullable): expert-choice scores [T, N] (each token's softmax over its N
// logits) are written instead of ids, gates and margin.
hipError_t launch_router(const moe_config& c, const void* h, const void* w_gate, const float* bias, float* logits,
                         int32_t* ids, float* gates, float* margin, hipStream_t s, const int32_t* replay = nullptr,
                         float* scores = nullptr);
hipError_t launch_topk(const moe_config& c, const float* logits, int32_t* ids, float* gates, float* margin,
                       hipStream_t s, const int32_t* replay = nullptr, float* scores = nullptr);

// ---- alignment (align.hip)
int align_chunk_routes();                       // routes per alignment chunk
size_t align_workspace_bytes(const moe_config& c);
// zero / nzero (nullable): words the scan kernel also sets to 0 (the GEMMs' work
// counters in the forward workspace), so no separate fill launch is needed
// stats_ready: the stats other than the padded row count were written already
// (by the reroute pass) and are left alone.
hipError_t launch_align(const moe_config& c, const int32_t* ids, uint8_t* kept, int32_t* sorted_ids,
                        int32_t* block_expert, int32_t* offsets, int32_t* num_padded, int32_t* stats,
                        void* ws, hipStream_t s, int32_t* zero = nullptr, int nzero = 0, bool stats_ready = false);

// ---- reroute overflow policy (reroute.hip)
// Workspace bytes of the reroute pass (besides the alignment's own).
size_t reroute_workspace_bytes(const moe_config& c);
// Capacity with rerouting, then the alignment of the routes as rerouted:
// route_expert [T*k] out = the expert each route runs (-1: none); logits [T, N]
// give each token's ranking for its candidates.  cap from the config (dropless:
// every valid route runs its own expert).
hipError_t launch_align_reroute(const moe_config& c, const int32_t* ids, const float* logits, int32_t* route_expert,
                                uint8_t* kept, int32_t* sorted_ids, int32_t* block_expert, int32_t* offsets,
                                int32_t* num_padded, int32_t* stats, void* ws, hipStream_t s,
                                int32_t* zero = nullptr, int nzero = 0);

// ---- expert-choice routing (expert_choice.hip)
inline bool expert_choice(const moe_config& c) { return c.routing == MOE_ROUTING_EXPERT_CHOICE; }
// Tokens each expert takes: min(floor(T*k*cf / N), T), cf = 1 for an unset (0/0) factor.
inline int ec_capacity(const moe_config& c) {
  long long num = c.cap_num, den = c.cap_den;
  if (num == 0 && den == 0) num = den = 1;
  const long long cap = ((long long)c.T * c.k * num) / ((long long)c.N * den);
  return (int)(cap < c.T ? cap : c.T);
}
// Rows of one expert's segment: its C picks rounded up to whole B-row blocks.
inline int ec_segment(const moe_config& c) { return (ec_capacity(c) + c.B - 1) / c.B * c.B; }
// Each expert's picks from scores [T, N]: tokens [N, C], slot [T, N], margin [N] (nullable).
hipError_t launch_ec_select(const moe_config& c, const float* scores, int32_t* tokens, int32_t* slot, float* margin,
                            hipStream_t s);
// Padded rows of the picks; zero / nzero as launch_align.
hipError_t launch_ec_align(const moe_config& c, const int32_t* tokens, const int32_t* slot, int32_t* sorted_ids,
                           int32_t* block_expert, int32_t* offsets, int32_t* num_padded, int32_t* stats,
                           hipStream_t s, int32_t* zero = nullptr, int nzero = 0);

// Compute units of the current device: queried once per device, then cached (api.hip).
hipError_t current_device_cus(int* cus);

// ---- expert FFN (ffn.hip)
// identity == true: one expert over T token rows (shared expert), offsets ignored.
// work (nullable): kGemmWorkWords zeroed ints per GEMM launch; with them the
// persistent workgroups claim tiles from per-XCD counters, without them each takes a
// fixed share.  The schedule changes no output bit.
constexpr int kGemmWorkWords = 8;
// w13_out (nullable): also store the gate and up projections, [rows, 2I] act dtype
// clk (nullable): MOE_CLOCK_SLOTS x 4 words, each persistent workgroup's clock stamps
hipError_t launch_gate_up(const moe_config& c, const void* h, const int32_t* sorted_ids, const int32_t* offsets,
                          const void* w13, const void* w13_scale, void* act, void* w13_out, bool identity,
                          hipStream_t s, int32_t* work = nullptr, uint64_t* clk = nullptr);
hipError_t launch_down(const moe_config& c, const void* act, const int32_t* sorted_ids, const int32_t* offsets,
                       const void* w2, const void* w2_scale, void* y, bool identity, hipStream_t s,
                       int32_t* work = nullptr, uint64_t* clk = nullptr);
// work: 2 * kGemmWorkWords ints (W13, then W2), or null
hipError_t launch_expert_ffn(const moe_config& c, const void* h, const int32_t* sorted_ids,
                             const int32_t* offsets, const void* w13, const void* w2, const void* w13_scale,
                             const void* w2_scale, void* act, void* w13_out, void* y, bool identity,
                             hipStream_t s, int32_t* work = nullptr);

// ---- combine (combine.hip)
hipError_t launch_combine(const moe_config& c, const void* y_route, const float* gates, const uint8_t* kept,
                          const void* shared_out, const void* residual, void* out, hipStream_t s);
// expert choice: y rows [N * segment, H], scores and slot [T, N]
hipError_t launch_combine_ec(const moe_config& c, const void* y_rows, const float* scores, const int32_t* slot,
                             const void* shared_out, const void* residual, void* out, hipStream_t s);

}  // namespace moe
