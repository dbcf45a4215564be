// Router: projection h . W_g^T to one fp32 logit per expert, then top-k with the
// lowest-index tie rule, renormalised softmax gates and the router margin.
//
// "Mixture-of-Experts Routing at Inference Time", "How sparse routing works" and
// "Worked example: a top-k router": W_g projects h to N logits; softmax; keep the
// top k; renormalise their gates.  "Mixture-of-experts routing & LLM
// repeatability": top-k is fixed by the scores and the tie rule; the margin is
// the gap between the k-th and (k+1)-th scores.
//
// Batch invariance ("Why temperature=0 Still Gives Different Answers: Batch
// Invariance", "How do I make LLM inference reproducible?", tier 2): each logit
// is reduced over fixed 32-wide K steps in ascending order inside a fixed
// quarter of H per wave, and the four quarters are added in a fixed order.
// Nothing depends on T or on the other tokens.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kRouterTokens = 16;   // tokens per workgroup (one 16-wide MFMA column block)
constexpr int kRouterWaves = 4;     // waves per workgroup, each owns a quarter of H

// bf16 projection on MFMA 16x16x32: D[expert][token] = sum_k W_g[expert][k] * h[token][k].
template <int NSUB>
__global__ __launch_bounds__(256) void router_logits_bf16(const __bf16* __restrict__ h,
                                                           const __bf16* __restrict__ wg,
                                                           const float* __restrict__ bias,
                                                           float* __restrict__ logits, int T, int H, int N) {
  __shared__ float part[kRouterWaves][NSUB * 16][kRouterTokens];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t0 = blockIdx.x * kRouterTokens;
  const int col = lane & 15, kq = (lane >> 4) * 8;
  const int tok = t0 + col;
  const int kspan = H / kRouterWaves;
  const int kbeg = wave * kspan;

  f32x4 acc[NSUB];
#pragma unroll
  for (int s = 0; s < NSUB; ++s) acc[s] = f32x4{0.f, 0.f, 0.f, 0.f};

  const bf16x8 zero8 = bf16x8{};
  const __bf16* hrow = h + (size_t)(tok < T ? tok : 0) * H + kq;
  const bool tok_ok = tok < T;
  for (int k0 = kbeg; k0 < kbeg + kspan; k0 += 32) {
    bf16x8 xb = tok_ok ? *reinterpret_cast<const bf16x8*>(hrow + k0) : zero8;
#pragma unroll
    for (int s = 0; s < NSUB; ++s) {
      const int e = s * 16 + col;
      bf16x8 wa = e < N ? *reinterpret_cast<const bf16x8*>(wg + (size_t)e * H + k0 + kq) : zero8;
      acc[s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa, xb, acc[s], 0, 0, 0);
    }
  }
  // lane holds token column (lane & 15), expert rows 4*(lane>>4) + r
#pragma unroll
  for (int s = 0; s < NSUB; ++s)
#pragma unroll
    for (int r = 0; r < 4; ++r) part[wave][s * 16 + (lane >> 4) * 4 + r][col] = acc[s][r];
  __syncthreads();
  for (int i = threadIdx.x; i < NSUB * 16 * kRouterTokens; i += blockDim.x) {
    const int e = i / kRouterTokens, t = i % kRouterTokens;
    if (e >= N || t0 + t >= T) continue;
    float v = part[0][e][t];
    v += part[1][e][t];
    v += part[2][e][t];
    v += part[3][e][t];
    if (bias) v += bias[e];
    logits[(size_t)(t0 + t) * N + e] = v;
  }
}

// fp32 projection: one thread per (token, expert), fmaf over H in ascending order.
__global__ __launch_bounds__(256) void router_logits_f32(const float* __restrict__ h, const float* __restrict__ wg,
                                                          const float* __restrict__ bias,
                                                          float* __restrict__ logits, int T, int H, int N) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (long)T * N) return;
  const int t = (int)(i / N), e = (int)(i % N);
  const float* x = h + (size_t)t * H;
  const float* w = wg + (size_t)e * H;
  float acc = 0.f;
  for (int k = 0; k < H; ++k) acc = fmaf(x[k], w[k], acc);
  if (bias) acc += bias[e];
  logits[i] = acc;
}

// Top-k over one token's N logits per wave.  Each lane holds experts lane + 64*i.
// k+1 rounds of a wave-wide max over (value, -index) keys give the ranked ids and
// the (k+1)-th logit for the margin.
constexpr int kTopkTokensPerBlock = 4;

__global__ __launch_bounds__(256) void topk_gates(const float* __restrict__ logits, int32_t* __restrict__ ids,
                                                   float* __restrict__ gates, float* __restrict__ margin,
                                                   int T, int N, int k, int renormalize) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * kTopkTokensPerBlock + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* lrow = logits + (size_t)t * N;
  float lv[4];
  uint64_t key[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane + 64 * i;
    lv[i] = e < N ? lrow[e] : 0.f;
    key[i] = e < N ? rank_key(lv[i], e) : 0ull;
  }
  const int rounds = k < N ? k + 1 : k;
  float sl[9];
  int sid[9];
#pragma unroll
  for (int j = 0; j < 9; ++j) {
    sl[j] = 0.f;
    sid[j] = 0;
    if (j < rounds) {
      uint64_t best = key[0];
#pragma unroll
      for (int i = 1; i < 4; ++i) best = key[i] > best ? key[i] : best;
      best = wave_max_u64(best);
      const int e = (int)(0xFFFFFFFFu - (uint32_t)best);
      const int owner = e & 63, slot = e >> 6;
      float mine = lv[0];
#pragma unroll
      for (int i = 1; i < 4; ++i) mine = slot == i ? lv[i] : mine;
      sl[j] = __shfl(mine, owner, kWave);
      sid[j] = e;
      if (lane == owner) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (i == slot) key[i] = 0ull;
      }
    }
  }
  // gates: weight_j = exp(l_j - l_0) (zero for a NaN logit), divided by the sum over
  // the k chosen in rank order, or by the sum over all N experts without renormalisation.
  const float l0 = sl[0];
  float w[8];
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    w[j] = 0.f;
    if (j < k) {
      w[j] = (sl[j] != sl[j]) ? 0.f : expf(sl[j] - l0);
      s += w[j];
    }
  }
  if (!renormalize) {
    float z = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = lane + 64 * i;
      if (e < N && lv[i] == lv[i]) z += expf(lv[i] - l0);
    }
    s = wave_sum_f32(z);
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (j < k && lane == j) {
      ids[(size_t)t * k + j] = sid[j];
      gates[(size_t)t * k + j] = w[j] / s;
    }
  }
  if (margin && lane == 0) {
    float m = __builtin_inff();
#pragma unroll
    for (int j = 1; j < 9; ++j)
      if (j == k && k < N) m = sl[j - 1] - sl[j];
    margin[t] = m;
  }
}

template <int NSUB>
hipError_t launch_router_bf16(const moe_config& c, const void* h, const void* wg, const float* bias, float* logits,
                              hipStream_t s) {
  dim3 grid(ceil_div(c.T, kRouterTokens));
  router_logits_bf16<NSUB><<<grid, 256, 0, s>>>((const __bf16*)h, (const __bf16*)wg, bias, logits, c.T, c.H, c.N);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_router_logits(const moe_config& c, const void* h, const void* w_gate, const float* bias,
                                float* logits, hipStream_t s) {
  if (c.act_dtype == MOE_F32) {
    const long n = (long)c.T * c.N;
    router_logits_f32<<<dim3((unsigned)((n + 255) / 256)), 256, 0, s>>>((const float*)h, (const float*)w_gate, bias,
                                                                        logits, c.T, c.H, c.N);
    return hipGetLastError();
  }
  switch (ceil_div(c.N, 16)) {
    case 1: return launch_router_bf16<1>(c, h, w_gate, bias, logits, s);
    case 2: return launch_router_bf16<2>(c, h, w_gate, bias, logits, s);
    case 3: return launch_router_bf16<3>(c, h, w_gate, bias, logits, s);
    case 4: return launch_router_bf16<4>(c, h, w_gate, bias, logits, s);
    case 5: return launch_router_bf16<5>(c, h, w_gate, bias, logits, s);
    case 6: return launch_router_bf16<6>(c, h, w_gate, bias, logits, s);
    case 7: return launch_router_bf16<7>(c, h, w_gate, bias, logits, s);
    case 8: return launch_router_bf16<8>(c, h, w_gate, bias, logits, s);
    case 9: return launch_router_bf16<9>(c, h, w_gate, bias, logits, s);
    case 10: return launch_router_bf16<10>(c, h, w_gate, bias, logits, s);
    case 11: return launch_router_bf16<11>(c, h, w_gate, bias, logits, s);
    case 12: return launch_router_bf16<12>(c, h, w_gate, bias, logits, s);
    case 13: return launch_router_bf16<13>(c, h, w_gate, bias, logits, s);
    case 14: return launch_router_bf16<14>(c, h, w_gate, bias, logits, s);
    case 15: return launch_router_bf16<15>(c, h, w_gate, bias, logits, s);
    default: return launch_router_bf16<16>(c, h, w_gate, bias, logits, s);
  }
}

hipError_t launch_topk(const moe_config& c, const float* logits, int32_t* ids, float* gates, float* margin,
                       hipStream_t s) {
  dim3 grid(ceil_div(c.T, kTopkTokensPerBlock));
  topk_gates<<<grid, 256, 0, s>>>(logits, ids, gates, margin, c.T, c.N, c.k, c.renormalize);
  return hipGetLastError();
}

}  // namespace moe
