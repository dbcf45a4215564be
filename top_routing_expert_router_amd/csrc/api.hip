// Host side of the C ABI declared in include/moe.h: argument validation,
// workspace layout, and the moe_forward composition on one stream.
// Validation runs before any HIP call, so every error path is host-only.
#include <string.h>

#include <atomic>
#include <mutex>

#include "common.h"
#include "kernels.h"

using namespace moe;

namespace moe {

// Per-device compute-unit counts, looked up on the first launch on each device (the
// persistent GEMMs and the router size their grids by it).  0 = not yet known.
namespace {
constexpr int kMaxCuDevices = 64;
std::atomic<int> g_cus[kMaxCuDevices];
}  // namespace

hipError_t current_device_cus(int* cus) {
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev >= 0 && dev < kMaxCuDevices) {
    const int known = g_cus[dev].load(std::memory_order_relaxed);
    if (known > 0) {
      *cus = known;
      return hipSuccess;
    }
  }
  int n = 0;
  err = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
  if (err != hipSuccess) return err;
  if (dev >= 0 && dev < kMaxCuDevices) g_cus[dev].store(n, std::memory_order_relaxed);
  *cus = n;
  return hipSuccess;
}

}  // namespace moe

// Scratch of moe_forward_noalloc: every intermediate of one forward pass, for callers that
// cannot allocate.  One copy per GPU, held until the process ends.  Host code never uses this
// name as an address (on the host it is only a stand-in for the symbol): the device address
// comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

moe_status check_config(const moe_config* c) {
  if (!c) return MOE_ERR_NULL_POINTER;
  if (c->struct_size < sizeof(moe_config)) return MOE_ERR_INVALID_CONFIG;
  if (c->T < 1 || c->T > 65536) return MOE_ERR_INVALID_CONFIG;
  if (c->H < 128 || c->H > 32768 || c->H % 128) return MOE_ERR_INVALID_CONFIG;
  if (c->I < 128 || c->I > 32768 || c->I % 128) return MOE_ERR_INVALID_CONFIG;
  if (c->N < 1 || c->N > 256) return MOE_ERR_INVALID_CONFIG;
  if (c->k < 1 || c->k > 8 || c->k > c->N) return MOE_ERR_INVALID_CONFIG;
  if (!(c->B == 8 || c->B == 16 || c->B == 32 || c->B == 64 || c->B == 128)) return MOE_ERR_INVALID_CONFIG;
  const bool dropless = c->cap_num == 0 && c->cap_den == 0;
  if (!dropless && (c->cap_num <= 0 || c->cap_den <= 0)) return MOE_ERR_INVALID_CONFIG;
  if (c->n_shared != 0 && c->n_shared != 1) return MOE_ERR_INVALID_CONFIG;
  if (c->renormalize != 0 && c->renormalize != 1) return MOE_ERR_INVALID_CONFIG;
  if (c->reroute_depth < 0 || c->reroute_depth > c->N - c->k) return MOE_ERR_INVALID_CONFIG;
  if (c->routing != MOE_ROUTING_TOKEN_CHOICE && c->routing != MOE_ROUTING_EXPERT_CHOICE) return MOE_ERR_INVALID_CONFIG;
  if (c->routing == MOE_ROUTING_EXPERT_CHOICE && c->reroute_depth != 0) return MOE_ERR_INVALID_CONFIG;
  const bool f32 = c->act_dtype == MOE_F32 && c->expert_dtype == MOE_F32 && c->scale_block == 0;
  const bool bf16 = c->act_dtype == MOE_BF16 && c->expert_dtype == MOE_BF16 && c->scale_block == 0;
  const bool fp8 = c->act_dtype == MOE_BF16 && c->expert_dtype == MOE_FP8_E4M3 && c->scale_block == 128;
  if (!(f32 || bf16 || fp8)) {
    const bool known = (c->act_dtype == MOE_F32 || c->act_dtype == MOE_BF16) &&
                       (c->expert_dtype >= MOE_F32 && c->expert_dtype <= MOE_FP8_E4M3);
    return known ? MOE_ERR_UNSUPPORTED : MOE_ERR_INVALID_CONFIG;
  }
  // the MFMA GEMMs address h and one expert's weights with 32-bit byte offsets
  if (!f32 && ((long)c->T * c->H >= (1L << 31) || 2L * c->I * c->H >= (1L << 31))) return MOE_ERR_INVALID_CONFIG;
  return MOE_OK;
}

size_t act_size(const moe_config& c) { return c.act_dtype == MOE_F32 ? 4 : 2; }
// padded row bound: token choice T*k + N*(B-1); expert choice exactly N segments
long p_max_of(const moe_config& c) {
  return expert_choice(c) ? (long)c.N * ec_segment(c) : (long)c.T * c.k + (long)c.N * (c.B - 1);
}
long n_blocks_of(const moe_config& c) { return (p_max_of(c) + c.B - 1) / c.B; }

size_t round_up(size_t x) { return (x + 255) & ~(size_t)255; }

// Regions of the moe_forward workspace, in order, each 256-byte aligned.
struct FwdLayout {
  size_t logits, ids, gates, margin, kept, rexp, scores, ctok, cslot, cmargin, sorted, blocks, offsets, npad, stats,
      align_ws, work, act, y, sact, sout, total;
};

FwdLayout forward_layout(const moe_config& c) {
  FwdLayout L{};
  const bool ec = expert_choice(c);
  const size_t T = c.T, N = c.N, R = ec ? 0 : (size_t)c.T * c.k, P = p_max_of(c), a = act_size(c);
  const size_t TN = ec ? T * N : 0, C = ec ? ec_capacity(c) : 0;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += round_up(bytes);
    return at;
  };
  L.logits = take(T * N * 4);
  L.ids = take(R * 4);
  L.gates = take(R * 4);
  L.margin = take(T * 4);
  L.kept = take(R);
  L.rexp = take(R * 4);
  L.scores = take(TN * 4);
  L.ctok = take(N * C * 4);
  L.cslot = take(TN * 4);
  L.cmargin = take(ec ? N * 4 : 0);
  L.sorted = take(P * 4);
  L.blocks = take(n_blocks_of(c) * 4);
  L.offsets = take((N + 1) * 4);
  L.npad = take(4);
  L.stats = take((N + MOE_STATS_EXTRA) * 4);
  L.align_ws = take(ec ? 0 : reroute_workspace_bytes(c) + round_up(align_workspace_bytes(c)));
  L.work = take(4 * kGemmWorkWords * 4);  // tile counters of the 4 expert GEMM launches
  L.act = take(P * (size_t)c.I * a);
  L.y = take((ec ? P : R) * (size_t)c.H * a);
  L.sact = c.n_shared ? take(T * (size_t)c.I * a) : o;
  L.sout = c.n_shared ? take(T * (size_t)c.H * a) : o;
  L.total = o;
  return L;
}

moe_status hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// A valid config with the given routing, else the error to return.
moe_status check_routing(const moe_config* c, bool want_expert_choice) {
  moe_status st = check_config(c);
  if (st != MOE_OK) return st;
  return expert_choice(*c) == want_expert_choice ? MOE_OK : MOE_ERR_UNSUPPORTED;
}

moe_status check_route_args(const moe_config& c, const void* h, const void* w_gate, const float* bias,
                            const float* logits, const int32_t* ids, const float* gates, const float* margin,
                            uint32_t flags) {
  if (flags & ~(uint32_t)(MOE_ROUTE_LOGITS_IN | MOE_ROUTE_IDS_IN | MOE_ROUTE_NO_LOGITS_OUT))
    return MOE_ERR_UNSUPPORTED;
  const bool in = flags & MOE_ROUTE_LOGITS_IN;
  const bool no_out = flags & MOE_ROUTE_NO_LOGITS_OUT;
  // no logits out: the bf16 projection keeps them on chip; the fp32 path stages them in
  // `logits` between its two kernels, and given logits are an input
  if (no_out && (in || c.act_dtype != MOE_BF16)) return MOE_ERR_UNSUPPORTED;
  if ((!logits && !no_out) || !ids || !gates) return MOE_ERR_NULL_POINTER;
  if (!in && (!h || !w_gate)) return MOE_ERR_NULL_POINTER;
  if ((logits && !aligned(logits, 4)) || !aligned(ids, 4) || !aligned(gates, 4) || (margin && !aligned(margin, 4)))
    return MOE_ERR_MISALIGNED;
  if (!in && (!aligned(h, 16) || !aligned(w_gate, 16) || (bias && !aligned(bias, 4)))) return MOE_ERR_MISALIGNED;
  return MOE_OK;
}

moe_status check_align_args(const int32_t* ids, const uint8_t* kept, const int32_t* sorted, const int32_t* blocks,
                            const int32_t* offsets, const int32_t* npad, const int32_t* stats, const void* ws) {
  if (!ids || !kept || !sorted || !blocks || !offsets || !npad || !ws) return MOE_ERR_NULL_POINTER;
  if (!aligned(ids, 4) || !aligned(sorted, 4) || !aligned(blocks, 4) || !aligned(offsets, 4) || !aligned(npad, 4) ||
      (stats && !aligned(stats, 4)) || !aligned(ws, 16))
    return MOE_ERR_MISALIGNED;
  return MOE_OK;
}

moe_status check_ffn_args(const moe_config& c, const void* h, const int32_t* sorted, const int32_t* offsets,
                          const void* w13, const void* w2, const void* s13, const void* s2, const void* act,
                          const void* w13_out, const void* y) {
  if (!h || !w13 || !w2 || !act || !y) return MOE_ERR_NULL_POINTER;
  if (sorted && !offsets) return MOE_ERR_NULL_POINTER;
  const bool fp8 = c.expert_dtype == MOE_FP8_E4M3;
  if (fp8 && (!s13 || !s2)) return MOE_ERR_NULL_POINTER;
  if (!aligned(h, 16) || !aligned(w13, 16) || !aligned(w2, 16) || !aligned(act, 16) || !aligned(y, 16) ||
      (w13_out && !aligned(w13_out, 16)))
    return MOE_ERR_MISALIGNED;
  if ((sorted && !aligned(sorted, 4)) || (offsets && !aligned(offsets, 4))) return MOE_ERR_MISALIGNED;
  if (fp8 && (!aligned(s13, 2) || !aligned(s2, 2))) return MOE_ERR_MISALIGNED;
  return MOE_OK;
}

moe_status check_combine_args(const void* y, const float* gates, const uint8_t* kept, const void* shared,
                              const void* residual, const void* out) {
  if (!y || !gates || !kept || !out) return MOE_ERR_NULL_POINTER;
  if (!aligned(y, 16) || !aligned(gates, 4) || !aligned(out, 16) || (shared && !aligned(shared, 16)) ||
      (residual && !aligned(residual, 16)))
    return MOE_ERR_MISALIGNED;
  return MOE_OK;
}

}  // namespace

extern "C" {

int32_t moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_status_str(moe_status s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_NULL_POINTER: return "MOE_ERR_NULL_POINTER: a required pointer is NULL";
    case MOE_ERR_INVALID_CONFIG: return "MOE_ERR_INVALID_CONFIG: config outside the supported envelope";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: dtype combination or flag not implemented";
    case MOE_ERR_MISALIGNED: return "MOE_ERR_MISALIGNED: pointer alignment rule violated";
    case MOE_ERR_WORKSPACE_TOO_SMALL: return "MOE_ERR_WORKSPACE_TOO_SMALL: workspace below moe_workspace_size";
    case MOE_ERR_HIP: return "MOE_ERR_HIP: a HIP runtime call or kernel launch failed";
    default: return "unknown moe_status";
  }
}

moe_status moe_validate_config(const moe_config* cfg) { return check_config(cfg); }

moe_status moe_align_sizes(const moe_config* cfg, int32_t* p_max, int32_t* n_blocks) {
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (!p_max || !n_blocks) return MOE_ERR_NULL_POINTER;
  *p_max = (int32_t)p_max_of(*cfg);
  *n_blocks = (int32_t)n_blocks_of(*cfg);
  return MOE_OK;
}

moe_status moe_workspace_size(const moe_config* cfg, int32_t op, size_t* bytes) {
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (!bytes) return MOE_ERR_NULL_POINTER;
  if (op == MOE_OP_ALIGN) {  // moe_align and moe_align_reroute (moe_align_expert_choice needs none)
    *bytes = expert_choice(*cfg) ? 0 : reroute_workspace_bytes(*cfg) + round_up(align_workspace_bytes(*cfg));
    return MOE_OK;
  }
  if (op == MOE_OP_FORWARD) {
    *bytes = forward_layout(*cfg).total;
    return MOE_OK;
  }
  return MOE_ERR_INVALID_CONFIG;
}

moe_status moe_route(const moe_config* cfg, const void* h, const void* w_gate, const float* logit_bias, float* logits,
                     int32_t* topk_ids, float* topk_gates, float* margin, uint32_t flags, void* stream) {
  moe_status st = check_routing(cfg, false);
  if (st != MOE_OK) return st;
  st = check_route_args(*cfg, h, w_gate, logit_bias, logits, topk_ids, topk_gates, margin, flags);
  if (st != MOE_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  // replay: the recorded ids are read, never written
  const int32_t* replay = (flags & MOE_ROUTE_IDS_IN) ? topk_ids : nullptr;
  int32_t* ids_out = replay ? nullptr : topk_ids;
  if (flags & MOE_ROUTE_LOGITS_IN)
    return hip_status(launch_topk(*cfg, logits, ids_out, topk_gates, margin, s, replay));
  return hip_status(launch_router(*cfg, h, w_gate, logit_bias, (flags & MOE_ROUTE_NO_LOGITS_OUT) ? nullptr : logits,
                                  ids_out, topk_gates, margin, s, replay));
}

moe_status moe_align(const moe_config* cfg, const int32_t* topk_ids, uint8_t* route_kept, int32_t* sorted_route_ids,
                     int32_t* block_expert, int32_t* expert_offsets, int32_t* num_padded, int32_t* stats, void* ws,
                     size_t ws_bytes, void* stream) {
  moe_status st = check_routing(cfg, false);
  if (st != MOE_OK) return st;
  st = check_align_args(topk_ids, route_kept, sorted_route_ids, block_expert, expert_offsets, num_padded, stats, ws);
  if (st != MOE_OK) return st;
  if (ws_bytes < align_workspace_bytes(*cfg)) return MOE_ERR_WORKSPACE_TOO_SMALL;
  return hip_status(launch_align(*cfg, topk_ids, route_kept, sorted_route_ids, block_expert, expert_offsets,
                                 num_padded, stats, ws, (hipStream_t)stream));
}

moe_status moe_align_reroute(const moe_config* cfg, const int32_t* topk_ids, const float* logits,
                             int32_t* route_expert, uint8_t* route_kept, int32_t* sorted_route_ids,
                             int32_t* block_expert, int32_t* expert_offsets, int32_t* num_padded, int32_t* stats,
                             void* ws, size_t ws_bytes, void* stream) {
  moe_status st = check_routing(cfg, false);
  if (st != MOE_OK) return st;
  st = check_align_args(topk_ids, route_kept, sorted_route_ids, block_expert, expert_offsets, num_padded, stats, ws);
  if (st != MOE_OK) return st;
  if (!logits || !route_expert) return MOE_ERR_NULL_POINTER;
  if (!aligned(logits, 4) || !aligned(route_expert, 4) || !aligned(ws, 256)) return MOE_ERR_MISALIGNED;
  if (ws_bytes < reroute_workspace_bytes(*cfg) + round_up(align_workspace_bytes(*cfg)))
    return MOE_ERR_WORKSPACE_TOO_SMALL;
  return hip_status(launch_align_reroute(*cfg, topk_ids, logits, route_expert, route_kept, sorted_route_ids,
                                         block_expert, expert_offsets, num_padded, stats, ws, (hipStream_t)stream));
}

moe_status moe_expert_ffn(const moe_config* cfg, const void* h, const int32_t* sorted_route_ids,
                          const int32_t* expert_offsets, const void* w13, const void* w2, const void* w13_scale,
                          const void* w2_scale, void* act, void* w13_out, void* y_out, void* stream) {
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  st = check_ffn_args(*cfg, h, sorted_route_ids, expert_offsets, w13, w2, w13_scale, w2_scale, act, w13_out, y_out);
  if (st != MOE_OK) return st;
  return hip_status(launch_expert_ffn(*cfg, h, sorted_route_ids, expert_offsets, w13, w2, w13_scale, w2_scale, act,
                                      w13_out, y_out, sorted_route_ids == nullptr, (hipStream_t)stream));
}

moe_status moe_expert_gate_up(const moe_config* cfg, const void* h, const int32_t* sorted_route_ids,
                              const int32_t* expert_offsets, const void* w13, const void* w13_scale, void* act,
                              void* w13_out, void* stream) {
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  const bool fp8 = cfg->expert_dtype == MOE_FP8_E4M3;
  if (!h || !w13 || !act || (sorted_route_ids && !expert_offsets) || (fp8 && !w13_scale)) return MOE_ERR_NULL_POINTER;
  if (!aligned(h, 16) || !aligned(w13, 16) || !aligned(act, 16) || (sorted_route_ids && !aligned(sorted_route_ids, 4)) ||
      (expert_offsets && !aligned(expert_offsets, 4)) || (fp8 && !aligned(w13_scale, 2)) ||
      (w13_out && !aligned(w13_out, 16)))
    return MOE_ERR_MISALIGNED;
  return hip_status(launch_gate_up(*cfg, h, sorted_route_ids, expert_offsets, w13, w13_scale, act, w13_out,
                                   sorted_route_ids == nullptr, (hipStream_t)stream));
}

moe_status moe_expert_down(const moe_config* cfg, const void* act, const int32_t* sorted_route_ids,
                           const int32_t* expert_offsets, const void* w2, const void* w2_scale, void* y_out,
                           void* stream) {
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  const bool fp8 = cfg->expert_dtype == MOE_FP8_E4M3;
  if (!act || !w2 || !y_out || (sorted_route_ids && !expert_offsets) || (fp8 && !w2_scale)) return MOE_ERR_NULL_POINTER;
  if (!aligned(act, 16) || !aligned(w2, 16) || !aligned(y_out, 16) || (sorted_route_ids && !aligned(sorted_route_ids, 4)) ||
      (expert_offsets && !aligned(expert_offsets, 4)) || (fp8 && !aligned(w2_scale, 2)))
    return MOE_ERR_MISALIGNED;
  return hip_status(launch_down(*cfg, act, sorted_route_ids, expert_offsets, w2, w2_scale, y_out,
                                sorted_route_ids == nullptr, (hipStream_t)stream));
}

moe_status moe_combine(const moe_config* cfg, const void* y_route, const float* topk_gates, const uint8_t* route_kept,
                       const void* shared_out, const void* residual, void* out, void* stream) {
  moe_status st = check_routing(cfg, false);
  if (st != MOE_OK) return st;
  st = check_combine_args(y_route, topk_gates, route_kept, shared_out, residual, out);
  if (st != MOE_OK) return st;
  return hip_status(launch_combine(*cfg, y_route, topk_gates, route_kept, shared_out, residual, out,
                                   (hipStream_t)stream));
}

moe_status moe_expert_choice_sizes(const moe_config* cfg, int32_t* capacity, int32_t* segment) {
  moe_status st = check_routing(cfg, true);
  if (st != MOE_OK) return st;
  if (!capacity || !segment) return MOE_ERR_NULL_POINTER;
  *capacity = ec_capacity(*cfg);
  *segment = ec_segment(*cfg);
  return MOE_OK;
}

moe_status moe_route_expert_choice(const moe_config* cfg, const void* h, const void* w_gate, const float* logit_bias,
                                   float* logits, float* scores, int32_t* choice_tokens, int32_t* choice_slot,
                                   float* choice_margin, uint32_t flags, void* stream) {
  moe_status st = check_routing(cfg, true);
  if (st != MOE_OK) return st;
  if (flags & ~(uint32_t)MOE_ROUTE_LOGITS_IN) return MOE_ERR_UNSUPPORTED;
  const bool in = flags & MOE_ROUTE_LOGITS_IN;
  if (!logits || !scores || !choice_slot || (!choice_tokens && ec_capacity(*cfg) > 0)) return MOE_ERR_NULL_POINTER;
  if (!in && (!h || !w_gate)) return MOE_ERR_NULL_POINTER;
  if (!aligned(logits, 4) || !aligned(scores, 4) || !aligned(choice_tokens, 4) || !aligned(choice_slot, 4) ||
      !aligned(choice_margin, 4))
    return MOE_ERR_MISALIGNED;
  if (!in && (!aligned(h, 16) || !aligned(w_gate, 16) || (logit_bias && !aligned(logit_bias, 4))))
    return MOE_ERR_MISALIGNED;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = in ? launch_topk(*cfg, logits, nullptr, nullptr, nullptr, s, nullptr, scores)
                    : launch_router(*cfg, h, w_gate, logit_bias, logits, nullptr, nullptr, nullptr, s, nullptr, scores);
  if (e == hipSuccess) e = launch_ec_select(*cfg, scores, choice_tokens, choice_slot, choice_margin, s);
  return hip_status(e);
}

moe_status moe_align_expert_choice(const moe_config* cfg, const int32_t* choice_tokens, const int32_t* choice_slot,
                                   int32_t* sorted_route_ids, int32_t* block_expert, int32_t* expert_offsets,
                                   int32_t* num_padded, int32_t* stats, void* stream) {
  moe_status st = check_routing(cfg, true);
  if (st != MOE_OK) return st;
  const bool rows = ec_capacity(*cfg) > 0;
  if ((rows && (!choice_tokens || !sorted_route_ids || !block_expert)) || !expert_offsets || !num_padded ||
      (stats && !choice_slot))
    return MOE_ERR_NULL_POINTER;
  if (!aligned(choice_tokens, 4) || !aligned(choice_slot, 4) || !aligned(sorted_route_ids, 4) ||
      !aligned(block_expert, 4) || !aligned(expert_offsets, 4) || !aligned(num_padded, 4) || !aligned(stats, 4))
    return MOE_ERR_MISALIGNED;
  return hip_status(launch_ec_align(*cfg, choice_tokens, choice_slot, sorted_route_ids, block_expert, expert_offsets,
                                    num_padded, stats, (hipStream_t)stream));
}

moe_status moe_combine_expert_choice(const moe_config* cfg, const void* y_rows, const float* scores,
                                     const int32_t* choice_slot, const void* shared_out, const void* residual,
                                     void* out, void* stream) {
  moe_status st = check_routing(cfg, true);
  if (st != MOE_OK) return st;
  if ((!y_rows && ec_capacity(*cfg) > 0) || !scores || !choice_slot || !out) return MOE_ERR_NULL_POINTER;
  if (!aligned(y_rows, 16) || !aligned(scores, 4) || !aligned(choice_slot, 4) || !aligned(out, 16) ||
      !aligned(shared_out, 16) || !aligned(residual, 16))
    return MOE_ERR_MISALIGNED;
  return hip_status(launch_combine_ec(*cfg, y_rows, scores, choice_slot, shared_out, residual, out,
                                     (hipStream_t)stream));
}

namespace {

// moe_forward and moe_forward_replay (replay: recorded expert ids, or null)
moe_status forward_impl(const moe_config* cfg, const moe_weights* wt, const void* h, const void* residual,
                        const int32_t* replay, void* out, const moe_trace* trace, void* ws, size_t ws_bytes,
                        void* stream) {
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  const moe_config& c = *cfg;
  if (!wt || !h || !out || !ws) return MOE_ERR_NULL_POINTER;
  if (!wt->w_gate || !wt->w13 || !wt->w2) return MOE_ERR_NULL_POINTER;
  const bool fp8 = c.expert_dtype == MOE_FP8_E4M3;
  if (fp8 && (!wt->w13_scale || !wt->w2_scale)) return MOE_ERR_NULL_POINTER;
  if (c.n_shared && (!wt->shared_w13 || !wt->shared_w2)) return MOE_ERR_NULL_POINTER;
  if (c.n_shared && fp8 && (!wt->shared_w13_scale || !wt->shared_w2_scale)) return MOE_ERR_NULL_POINTER;
  if (!aligned(h, 16) || !aligned(out, 16) || (residual && !aligned(residual, 16)) || !aligned(ws, 256) ||
      !aligned(wt->w_gate, 16) || !aligned(wt->w13, 16) || !aligned(wt->w2, 16) ||
      (wt->logit_bias && !aligned(wt->logit_bias, 4)) ||
      (c.n_shared && (!aligned(wt->shared_w13, 16) || !aligned(wt->shared_w2, 16))))
    return MOE_ERR_MISALIGNED;
  const FwdLayout L = forward_layout(c);
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE_TOO_SMALL;
  char* base = (char*)ws;
  moe_trace tr{};
  if (trace) tr = *trace;
  auto pick = [&](void* user, size_t off) -> void* { return user ? user : (void*)(base + off); };
  float* logits = (float*)pick(tr.logits, L.logits);
  int32_t* ids = replay ? const_cast<int32_t*>(replay) : (int32_t*)pick(tr.topk_ids, L.ids);
  float* gates = (float*)pick(tr.topk_gates, L.gates);
  float* margin = (float*)pick(tr.margin, L.margin);
  uint8_t* kept = (uint8_t*)pick(tr.route_kept, L.kept);
  int32_t* sorted = (int32_t*)pick(tr.sorted_route_ids, L.sorted);
  int32_t* blocks = (int32_t*)pick(tr.block_expert, L.blocks);
  int32_t* offsets = (int32_t*)pick(tr.expert_offsets, L.offsets);
  int32_t* npad = (int32_t*)pick(tr.num_padded, L.npad);
  int32_t* stats = (int32_t*)pick(tr.stats, L.stats);
  void* act = pick(tr.act, L.act);
  void* y = pick(tr.y_route, L.y);
  int32_t* work = (int32_t*)(base + L.work);  // zeroed by the alignment scan, used by the GEMMs
  int32_t* rexp = (int32_t*)pick(tr.route_expert, L.rexp);
  const bool reroute = c.reroute_depth > 0 && !(c.cap_num == 0 && c.cap_den == 0);
  if (!aligned(rexp, 4)) return MOE_ERR_MISALIGNED;
  if (!aligned(logits, 4) || !aligned(ids, 4) || !aligned(gates, 4) || !aligned(margin, 4) || !aligned(sorted, 4) ||
      !aligned(blocks, 4) || !aligned(offsets, 4) || !aligned(npad, 4) || !aligned(stats, 4) || !aligned(act, 16) ||
      !aligned(y, 16) || (tr.w13_out && !aligned(tr.w13_out, 16)) || !aligned(tr.gemm_clocks, 8))
    return MOE_ERR_MISALIGNED;

  hipStream_t s = (hipStream_t)stream;
  // stage events of the trace (nullable): recorded between the stages on this stream
  auto mark = [&](int i) -> hipError_t {
    return tr.stage_events && tr.stage_events[i] ? hipEventRecord((hipEvent_t)tr.stage_events[i], s) : hipSuccess;
  };
  // W13 then W2 of the routed experts, the shared expert, each followed by its event
  auto expert_stages = [&](hipError_t e, const void* shared_out_buf, const void** shared_out) -> hipError_t {
    if (e == hipSuccess)
      e = launch_gate_up(c, h, sorted, offsets, wt->w13, wt->w13_scale, act, tr.w13_out, false, s, work,
                         tr.gemm_clocks);
    if (e == hipSuccess) e = mark(3);
    if (e == hipSuccess)
      e = launch_down(c, act, sorted, offsets, wt->w2, wt->w2_scale, y, false, s, work + kGemmWorkWords,
                      tr.gemm_clocks ? tr.gemm_clocks + 4 * MOE_CLOCK_SLOTS : nullptr);
    if (e == hipSuccess) e = mark(4);
    if (e == hipSuccess && c.n_shared) {
      e = launch_expert_ffn(c, h, nullptr, nullptr, wt->shared_w13, wt->shared_w2, wt->shared_w13_scale,
                            wt->shared_w2_scale, base + L.sact, nullptr, (void*)shared_out_buf, true, s,
                            work + 2 * kGemmWorkWords);
      *shared_out = shared_out_buf;
    }
    if (e == hipSuccess) e = mark(5);
    return e;
  };
  if (expert_choice(c)) {
    float* scores = (float*)pick(tr.scores, L.scores);
    int32_t* ctok = (int32_t*)pick(tr.choice_tokens, L.ctok);
    int32_t* cslot = (int32_t*)pick(tr.choice_slot, L.cslot);
    float* cmargin = (float*)pick(tr.choice_margin, L.cmargin);
    if (!aligned(scores, 4) || !aligned(ctok, 4) || !aligned(cslot, 4) || !aligned(cmargin, 4))
      return MOE_ERR_MISALIGNED;
    hipError_t e = mark(0);
    if (e == hipSuccess)
      e = launch_router(c, h, wt->w_gate, wt->logit_bias, logits, nullptr, nullptr, nullptr, s, nullptr, scores);
    if (e == hipSuccess) e = launch_ec_select(c, scores, ctok, cslot, cmargin, s);
    if (e == hipSuccess) e = mark(1);
    if (e == hipSuccess)
      e = launch_ec_align(c, ctok, cslot, sorted, blocks, offsets, npad, stats, s, work, 4 * kGemmWorkWords);
    if (e == hipSuccess) e = mark(2);
    const void* shared_out = nullptr;
    e = expert_stages(e, base + L.sout, &shared_out);
    if (e == hipSuccess) e = launch_combine_ec(c, y, scores, cslot, shared_out, residual, out, s);
    if (e == hipSuccess) e = mark(6);
    return hip_status(e);
  }
  hipError_t e = mark(0);
  if (e == hipSuccess)
    e = launch_router(c, h, wt->w_gate, wt->logit_bias, logits, replay ? nullptr : ids, gates, margin, s, replay);
  if (e == hipSuccess) e = mark(1);
  if (e == hipSuccess)
    e = reroute ? launch_align_reroute(c, ids, logits, rexp, kept, sorted, blocks, offsets, npad, stats,
                                       base + L.align_ws, s, work, 4 * kGemmWorkWords)
                : launch_align(c, ids, kept, sorted, blocks, offsets, npad, stats,
                               base + L.align_ws + reroute_workspace_bytes(c), s, work, 4 * kGemmWorkWords);
  if (e == hipSuccess) e = mark(2);
  const void* shared_out = nullptr;
  e = expert_stages(e, base + L.sout, &shared_out);
  if (e == hipSuccess) e = launch_combine(c, y, gates, kept, shared_out, residual, out, s);
  if (e == hipSuccess) e = mark(6);
  return hip_status(e);
}

}  // namespace

moe_status moe_forward(const moe_config* cfg, const moe_weights* wt, const void* h, const void* residual, void* out,
                       const moe_trace* trace, void* ws, size_t ws_bytes, void* stream) {
  return forward_impl(cfg, wt, h, residual, nullptr, out, trace, ws, ws_bytes, stream);
}

moe_status moe_routing_health_from_stats(const moe_config* cfg, const int32_t* stats, moe_routing_health* out) {
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (!stats || !out) return MOE_ERR_NULL_POINTER;
  const int N = cfg->N;
  const int32_t* x = stats + N;
  long total = 0;
  int32_t mx = 0, mn = 0;
  for (int e = 0; e < N; ++e) {
    if (stats[e] < 0) return MOE_ERR_INVALID_CONFIG;
    total += stats[e];
    mx = e == 0 || stats[e] > mx ? stats[e] : mx;
    mn = e == 0 || stats[e] < mn ? stats[e] : mn;
  }
  if (x[MOE_STAT_KEPT] < 0 || x[MOE_STAT_DROPPED] < 0 || x[MOE_STAT_INVALID] < 0 || x[MOE_STAT_CAPACITY] < -1 ||
      x[MOE_STAT_REROUTED] < 0 || x[MOE_STAT_UNPICKED] < 0 || total > INT32_MAX)
    return MOE_ERR_INVALID_CONFIG;
  moe_routing_health r{};
  r.total_routes = (int32_t)total;
  r.max_expert_load = mx;
  r.min_expert_load = mn;
  r.dropped_routes = x[MOE_STAT_DROPPED];
  r.kept_routes = x[MOE_STAT_KEPT];
  r.invalid_routes = x[MOE_STAT_INVALID];
  r.capacity = x[MOE_STAT_CAPACITY];
  r.rerouted_routes = x[MOE_STAT_REROUTED];
  r.unpicked_tokens = x[MOE_STAT_UNPICKED];
  // imbalance = largest load over the mean load of the N experts; drops over all routed
  r.imbalance_ratio = total ? (double)mx * N / (double)total : 0.0;
  r.drop_fraction = total ? (double)r.dropped_routes / (double)total : 0.0;
  *out = r;
  return MOE_OK;
}

namespace {

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxScratchDevices];  // device address of `scratch` on each device, once looked up

// The device address of this device's `scratch` (looked up with the device current), or null.
void* scratch_on(int dev) {
  if (dev < 0 || dev >= kMaxScratchDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch[dev] = p;
  }
  return g_scratch[dev];
}

}  // namespace

moe_status moe_forward_noalloc(const moe_config* cfg, const moe_weights* wt, const void* h, const void* residual,
                               void* out, const moe_trace* trace, void* stream) {
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (forward_layout(*cfg).total > (size_t)MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE_TOO_SMALL;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
  void* ws = scratch_on(dev);
  if (ws == nullptr) return MOE_ERR_HIP;
  // the tile counters the GEMMs claim from are cleared by the alignment kernel inside the
  // forward; nothing else in the scratch is read before it is written
  return forward_impl(cfg, wt, h, residual, nullptr, out, trace, ws, (size_t)MOE_NOALLOC_SCRATCH_BYTES, stream);
}

moe_status moe_forward_replay(const moe_config* cfg, const moe_weights* wt, const void* h, const void* residual,
                              const int32_t* replay_ids, void* out, const moe_trace* trace, void* ws,
                              size_t ws_bytes, void* stream) {
  moe_status st = check_routing(cfg, false);
  if (st != MOE_OK) return st;
  if (!replay_ids) return MOE_ERR_NULL_POINTER;
  if (!aligned(replay_ids, 4)) return MOE_ERR_MISALIGNED;
  return forward_impl(cfg, wt, h, residual, replay_ids, out, trace, ws, ws_bytes, stream);
}

}  // extern "C"
