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
hipError_t launch_router(const moe_config& c, const void* h, const void* w_gate, const float* bias, float* logits,
                         int32_t* ids, float* gates, float* margin, hipStream_t s, const int32_t* replay = nullptr);
hipError_t launch_topk(const moe_config& c, const float* logits, int32_t* ids, float* gates, float* margin,
                       hipStream_t s, const int32_t* replay = nullptr);

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

// ---- expert FFN (ffn.hip)
// identity == true: one expert over T token rows (shared expert), offsets ignored.
// work (nullable): kGemmWorkWords zeroed ints per GEMM launch; with them the
// persistent workgroups claim tiles from per-XCD counters, without them each takes a
// fixed share.  The schedule changes no output bit.
constexpr int kGemmWorkWords = 8;
hipError_t launch_gate_up(const moe_config& c, const void* h, const int32_t* sorted_ids, const int32_t* offsets,
                          const void* w13, const void* w13_scale, void* act, bool identity, hipStream_t s,
                          int32_t* work = nullptr);
hipError_t launch_down(const moe_config& c, const void* act, const int32_t* sorted_ids, const int32_t* offsets,
                       const void* w2, const void* w2_scale, void* y, bool identity, hipStream_t s,
                       int32_t* work = nullptr);
// work: 2 * kGemmWorkWords ints (W13, then W2), or null
hipError_t launch_expert_ffn(const moe_config& c, const void* h, const int32_t* sorted_ids,
                             const int32_t* offsets, const void* w13, const void* w2, const void* w13_scale,
                             const void* w2_scale, void* act, void* y, bool identity, hipStream_t s,
                             int32_t* work = nullptr);

// ---- combine (combine.hip)
hipError_t launch_combine(const moe_config& c, const void* y_route, const float* gates, const uint8_t* kept,
                          const void* shared_out, const void* residual, void* out, hipStream_t s);

}  // namespace moe
