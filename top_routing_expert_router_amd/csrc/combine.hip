// Gate-weighted combine into the residual stream.
//
// "Mixture-of-experts routing & LLM repeatability": output = sum over the chosen
// experts of gate[e] * expert[e](h), returned to the residual stream.
// "Mixture-of-Experts Routing at Inference Time", "The hard part" (Figure 2): a
// dropped route contributes nothing; a fully dropped token carries h alone.
//
// out[t] = round(((sum over kept j ascending of gate[t,j] * y[t*k+j]) + shared[t]) + residual[t])
// in fp32 with fmaf for the weighted terms, in exactly this order, one rounding.
// The accumulator starts at -0.0 (the IEEE additive identity), so a token with no
// kept route and no shared expert outputs its residual bit for bit, -0 included.
// Each thread owns 8 consecutive columns of one token (16-byte bf16 accesses).
// A route whose kept flag is 0 contributes nothing: its y row (allocated, never
// written) is loaded but not added.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

template <typename T>
struct Vec8;
template <>
struct Vec8<__bf16> {
  typedef __bf16 type __attribute__((ext_vector_type(8)));
};
template <>
struct Vec8<float> {
  typedef float type __attribute__((ext_vector_type(8)));
};

constexpr int kColsPerThread = 8;
constexpr int kThreads = 256;
constexpr int kColsPerBlock = kColsPerThread * kThreads;

// One workgroup per (token, 2048-column slice): the token's gates and kept flags
// are uniform (one per lane, read back with readlane); every y row is loaded
// (all rows are allocated) and the kept flag selects whether it enters the sum, so
// all loads of a thread are in flight together.
template <typename T, int K>
__global__ __launch_bounds__(kThreads) void combine_rows(const T* __restrict__ y, const float* __restrict__ gates,
                                                          const uint8_t* __restrict__ kept, const T* __restrict__ shared,
                                                          const T* __restrict__ residual, T* __restrict__ out, int H,
                                                          int slices) {
  typedef typename Vec8<T>::type V;
  const int t = blockIdx.x / slices;
  const long col = (long)(blockIdx.x % slices) * kColsPerBlock + threadIdx.x * kColsPerThread;
  if (col >= H) return;
  // the token's k gates and kept flags, lane j holding route j, loaded before the rows
  // (a flag loaded where it is used waits for every row load issued before it)
  const int jl = (int)(threadIdx.x & 63) < K ? (int)(threadIdx.x & 63) : 0;
  const float g_lane = gates[(long)t * K + jl];
  const int on_lane = kept[(long)t * K + jl];
  V yv[K];
#pragma unroll
  for (int j = 0; j < K; ++j) yv[j] = *reinterpret_cast<const V*>(y + ((long)t * K + j) * H + col);
  V sv, rv;
  if (shared) sv = *reinterpret_cast<const V*>(shared + (long)t * H + col);
  if (residual) rv = *reinterpret_cast<const V*>(residual + (long)t * H + col);
  float acc[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) acc[q] = -0.0f;
#pragma unroll
  for (int j = 0; j < K; ++j) {
    const bool on = __builtin_amdgcn_readlane(on_lane, j) != 0;
    const float g = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(g_lane), j));
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const float f = fmaf(g, (float)yv[j][q], acc[q]);
      acc[q] = on ? f : acc[q];
    }
  }
  if (shared) {
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] += (float)sv[q];
  }
  if (residual) {
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] += (float)rv[q];
  }
  V o;
#pragma unroll
  for (int q = 0; q < 8; ++q) o[q] = cvt_act<T>(acc[q]);
  *reinterpret_cast<V*>(out + (long)t * H + col) = o;
}

// Expert choice: out[t] = round(((sum over the experts e that picked t, ascending, of
// score[t, e] * y[e * Cp + slot[t, e]]) + shared[t]) + residual[t]), fmaf per term in
// that order, one rounding ("Mixture-of-experts routing & LLM repeatability", paragraph
// on expert-choice routing: the gate of a pick is the token's score for that expert).
// The workgroup first lists its token's picks in LDS (thread e looks at expert e; ballot
// prefix counts keep ascending expert order), then loads the picked rows eight at a
// time, so a token's few picks among many experts are in flight together.
template <typename T>
__global__ __launch_bounds__(kThreads) void combine_ec_rows(const T* __restrict__ y, const float* __restrict__ scores,
                                                             const int32_t* __restrict__ slot,
                                                             const T* __restrict__ shared,
                                                             const T* __restrict__ residual, T* __restrict__ out,
                                                             int H, int N, int C, int Cp, int slices) {
  typedef typename Vec8<T>::type V;
  __shared__ int s_row[kThreads];
  __shared__ float s_gate[kThreads];
  __shared__ int s_cnt[kThreads / kWave];
  const int t = blockIdx.x / slices;
  const long col = (long)(blockIdx.x % slices) * kColsPerBlock + threadIdx.x * kColsPerThread;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  int pos = tid < N ? slot[(long)t * N + tid] : -1;  // N <= kThreads
  if (pos >= C) pos = -1;                            // slots are < C; anything else is not a pick
  const bool picked = pos >= 0;
  const uint64_t bal = __ballot(picked);
  if (lane == 0) s_cnt[wave] = __popcll(bal);
  __syncthreads();
  int before = 0, total = 0;
#pragma unroll
  for (int w = 0; w < kThreads / kWave; ++w) {
    before += w < wave ? s_cnt[w] : 0;
    total += s_cnt[w];
  }
  if (picked) {
    const int i = before + __popcll(bal & ((1ull << lane) - 1ull));
    s_row[i] = tid * Cp + pos;
    s_gate[i] = scores[(long)t * N + tid];
  }
  __syncthreads();
  if (col >= H) return;
  float acc[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) acc[q] = -0.0f;
  for (int i0 = 0; i0 < total; i0 += 8) {
    V yv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (i0 + j < total) yv[j] = *reinterpret_cast<const V*>(y + (long)s_row[i0 + j] * H + col);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (i0 + j < total) {
        const float g = s_gate[i0 + j];
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[q] = fmaf(g, (float)yv[j][q], acc[q]);
      }
    }
  }
  if (shared) {
    const V sv = *reinterpret_cast<const V*>(shared + (long)t * H + col);
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] += (float)sv[q];
  }
  if (residual) {
    const V rv = *reinterpret_cast<const V*>(residual + (long)t * H + col);
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] += (float)rv[q];
  }
  V o;
#pragma unroll
  for (int q = 0; q < 8; ++q) o[q] = cvt_act<T>(acc[q]);
  *reinterpret_cast<V*>(out + (long)t * H + col) = o;
}

}  // namespace

hipError_t launch_combine(const moe_config& c, const void* y_route, const float* gates, const uint8_t* kept,
                          const void* shared_out, const void* residual, void* out, hipStream_t s) {
  const int slices = ceil_div(c.H, kColsPerBlock);
  const dim3 grid((unsigned)c.T * slices);
  auto go = [&](auto kt) {
    constexpr int K = decltype(kt)::value;
    if (c.act_dtype == MOE_F32)
      combine_rows<float, K><<<grid, kThreads, 0, s>>>((const float*)y_route, gates, kept, (const float*)shared_out,
                                                       (const float*)residual, (float*)out, c.H, slices);
    else
      combine_rows<__bf16, K><<<grid, kThreads, 0, s>>>((const __bf16*)y_route, gates, kept,
                                                        (const __bf16*)shared_out, (const __bf16*)residual,
                                                        (__bf16*)out, c.H, slices);
  };
  switch (c.k) {  // 1 <= k <= 8 (checked with the config)
    case 1: go(std::integral_constant<int, 1>{}); break;
    case 2: go(std::integral_constant<int, 2>{}); break;
    case 3: go(std::integral_constant<int, 3>{}); break;
    case 4: go(std::integral_constant<int, 4>{}); break;
    case 5: go(std::integral_constant<int, 5>{}); break;
    case 6: go(std::integral_constant<int, 6>{}); break;
    case 7: go(std::integral_constant<int, 7>{}); break;
    default: go(std::integral_constant<int, 8>{}); break;
  }
  return hipGetLastError();
}

}  // namespace moe

namespace moe {

hipError_t launch_combine_ec(const moe_config& c, const void* y_rows, const float* scores, const int32_t* slot,
                             const void* shared_out, const void* residual, void* out, hipStream_t s) {
  const int slices = ceil_div(c.H, kColsPerBlock);
  const dim3 grid((unsigned)c.T * slices);
  const int Cp = ec_segment(c);
  if (c.act_dtype == MOE_F32) {
    combine_ec_rows<float><<<grid, kThreads, 0, s>>>((const float*)y_rows, scores, slot, (const float*)shared_out,
                                                     (const float*)residual, (float*)out, c.H, c.N, ec_capacity(c), Cp,
                                                     slices);
  } else {
    combine_ec_rows<__bf16><<<grid, kThreads, 0, s>>>((const __bf16*)y_rows, scores, slot,
                                                      (const __bf16*)shared_out, (const __bf16*)residual,
                                                      (__bf16*)out, c.H, c.N, ec_capacity(c), Cp, slices);
  }
  return hipGetLastError();
}

}  // namespace moe
