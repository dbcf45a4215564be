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
// Each thread owns 8 consecutive columns of one token in each of two 2048-column halves of
// a 4096-column slice (16-byte bf16 accesses, each wave instruction 1 KB contiguous).
// A route whose kept flag is 0 contributes nothing.  Without a capacity limit every valid
// route is kept, and the y rows of all routes are loaded together with the flags (a row
// whose flag is 0 -- an invalid replayed id -- is loaded but not added); with one, the
// flags are read first and only kept routes' rows are loaded.
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
constexpr int kColsPerBlock = kColsPerThread * kThreads;  // expert-choice combine: 2048 columns
constexpr int kChunks = 2;                                 // token-choice combine: 2 x 2048 columns
constexpr int kColsPerSlice = kColsPerBlock * kChunks;

// One workgroup per (token, 4096-column slice).  The token's k gates and kept flags are
// uniform (one per lane, read back with readlane).  Rows are read with buffer loads over
// the token's own rows: a column past H, or a row left out, is an offset past the
// resource, which reads zeros and no memory -- so no load sits under a branch (hipcc
// waits for every load in flight at the joins of such branches).  DROPS = false: every y
// row is loaded together with the flags, and a flag selects whether its row enters the
// sum.  DROPS = true (a capacity limit, where many routes may be dropped): one wait for
// the flags, then only the kept routes' rows are read.
template <typename T, int K, bool DROPS>
__global__ __launch_bounds__(kThreads) void combine_rows(const T* __restrict__ y, const float* __restrict__ gates,
                                                          const uint8_t* __restrict__ kept, const T* __restrict__ shared,
                                                          const T* __restrict__ residual, T* __restrict__ out, int H,
                                                          int slices) {
  typedef typename Vec8<T>::type V;
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  constexpr int NP = sizeof(V) / 16;  // 16-byte pieces per 8 columns
  const int t = blockIdx.x / slices;
  const int slice = blockIdx.x % slices;
  int col[kChunks];
#pragma unroll
  for (int c = 0; c < kChunks; ++c) col[c] = slice * kColsPerSlice + c * kColsPerBlock + threadIdx.x * kColsPerThread;
  // the token's k gates and kept flags, lane j holding route j: with drops read first (they
  // decide which rows are read), else after the rows are requested (vmcnt counts in order,
  // so waiting for a flag loaded first would hold back the row loads issued behind it)
  const int jl = (int)(threadIdx.x & 63) < K ? (int)(threadIdx.x & 63) : 0;
  float g_lane = 0.f;
  int on_lane = 0;
  if constexpr (DROPS) {
    g_lane = gates[(long)t * K + jl];
    on_lane = kept[(long)t * K + jl];
  }
  const uint32_t row_bytes = (uint32_t)H * sizeof(T);
  const __amdgpu_buffer_rsrc_t ry = __builtin_amdgcn_make_buffer_rsrc((void*)(y + (long)t * K * H), (short)0,
                                                                      (int)(K * row_bytes), kRawBufferFlags);
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)(shared ? shared + (long)t * H : y),
                                                                      (short)0, shared ? (int)row_bytes : 0,
                                                                      kRawBufferFlags);
  const __amdgpu_buffer_rsrc_t rr = __builtin_amdgcn_make_buffer_rsrc((void*)(residual ? residual + (long)t * H : y),
                                                                      (short)0, residual ? (int)row_bytes : 0,
                                                                      kRawBufferFlags);
  const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc((void*)(out + (long)t * H), (short)0,
                                                                      (int)row_bytes, kRawBufferFlags);
  const bool has_shared = shared != nullptr, has_residual = residual != nullptr;
  bool on[K];
  if constexpr (DROPS) {
#pragma unroll
    for (int j = 0; j < K; ++j) on[j] = __builtin_amdgcn_readlane(on_lane, j) != 0;
  }
  auto load8 = [&](__amdgpu_buffer_rsrc_t r, uint32_t off) {
    V v;
    u32x4 p[NP];
#pragma unroll
    for (int i = 0; i < NP; ++i)
      p[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off + 16u * i, 0, 0));
    __builtin_memcpy(&v, p, sizeof(V));
    return v;
  };
  V yv[K][kChunks], sv[kChunks], rv[kChunks];
#pragma unroll
  for (int c = 0; c < kChunks; ++c) {
    const uint32_t coff = col[c] < H ? (uint32_t)col[c] * sizeof(T) : kBufferOutOfRange;
#pragma unroll
    for (int j = 0; j < K; ++j)
      yv[j][c] = load8(ry, (DROPS && !on[j]) || col[c] >= H ? kBufferOutOfRange : j * row_bytes + coff);
    sv[c] = load8(rs, coff);
    rv[c] = load8(rr, coff);
  }
  if constexpr (!DROPS) {
    __builtin_amdgcn_sched_barrier(0);  // the row loads stay ahead of the flag loads
    g_lane = gates[(long)t * K + jl];
    on_lane = kept[(long)t * K + jl];
#pragma unroll
    for (int j = 0; j < K; ++j) on[j] = __builtin_amdgcn_readlane(on_lane, j) != 0;
  }
#pragma unroll
  for (int c = 0; c < kChunks; ++c) {
    float acc[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] = -0.0f;
#pragma unroll
    for (int j = 0; j < K; ++j) {
      const float g = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(g_lane), j));
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const float f = fmaf(g, (float)yv[j][c][q], acc[q]);
        acc[q] = on[j] ? f : acc[q];
      }
    }
    // absent terms add nothing (selects, not branches, so no load sinks under a branch;
    // adding a zero would turn an accumulator of -0 into +0)
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const float f = acc[q] + (float)sv[c][q];
      acc[q] = has_shared ? f : acc[q];
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const float f = acc[q] + (float)rv[c][q];
      acc[q] = has_residual ? f : acc[q];
    }
    V o;
#pragma unroll
    for (int q = 0; q < 8; ++q) o[q] = cvt_act<T>(acc[q]);
    // a buffer store past the row's end writes nothing: no branch here either
    const uint32_t ooff = col[c] < H ? (uint32_t)col[c] * sizeof(T) : kBufferOutOfRange;
    u32x4 p[NP];
    __builtin_memcpy(p, &o, sizeof(V));
#pragma unroll
    for (int i = 0; i < NP; ++i)
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned, p[i]), ro,
                                             ooff + 16u * i, 0, 0);
  }
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
  const int slices = ceil_div(c.H, kColsPerSlice);
  const dim3 grid((unsigned)c.T * slices);
  const bool drops = !(c.cap_num == 0 && c.cap_den == 0);
  auto go = [&](auto kt) {
    constexpr int K = decltype(kt)::value;
    auto run = [&](auto dt) {
      constexpr bool D = decltype(dt)::value;
      if (c.act_dtype == MOE_F32)
        combine_rows<float, K, D><<<grid, kThreads, 0, s>>>((const float*)y_route, gates, kept,
                                                            (const float*)shared_out, (const float*)residual,
                                                            (float*)out, c.H, slices);
      else
        combine_rows<__bf16, K, D><<<grid, kThreads, 0, s>>>((const __bf16*)y_route, gates, kept,
                                                             (const __bf16*)shared_out, (const __bf16*)residual,
                                                             (__bf16*)out, c.H, slices);
    };
    if (drops)
      run(std::true_type{});
    else
      run(std::false_type{});
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
