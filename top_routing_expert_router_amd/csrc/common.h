// Shared device/host helpers for the MI355X (gfx950) MoE layer kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

constexpr int kWave = 64;  // CDNA wavefront width

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Round-to-nearest-even float -> bf16 (gfx950 has a hardware convert for this).
__device__ __forceinline__ __bf16 to_bf16(float x) { return (__bf16)x; }
__device__ __forceinline__ float from_bf16(__bf16 x) { return (float)x; }

__device__ __forceinline__ uint16_t bf16_bits(__bf16 x) { return __builtin_bit_cast(uint16_t, x); }

// Load/store of one activation element as fp32, for the two activation types.
template <typename T> __device__ __forceinline__ float ld_act(const T* p);
template <> __device__ __forceinline__ float ld_act<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ float ld_act<__bf16>(const __bf16* p) { return (float)*p; }

template <typename T> __device__ __forceinline__ T cvt_act(float x);
template <> __device__ __forceinline__ float cvt_act<float>(float x) { return x; }
template <> __device__ __forceinline__ __bf16 cvt_act<__bf16>(float x) { return (__bf16)x; }

// silu(x) = x / (1 + e^-x), fp32, accurate expf and IEEE division (fp32 outputs).
__device__ __forceinline__ float silu_f32(float x) { return x / (1.0f + expf(-x)); }

// silu for results that are rounded to bf16 next: hardware exp2 and reciprocal
// (each within ~1 fp32 ulp, far below the bf16 rounding that follows).
// Large negative x: e^-x = inf, rcp(inf) = 0, x * 0 = -0.
__device__ __forceinline__ float silu_fast(float x) { return x * __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }

// Order-preserving 32-bit key of a float: larger float -> larger key; -0 and +0
// share a key; every NaN maps to 0, below -inf.
__device__ __forceinline__ uint32_t float_order_key(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if (f != f) return 0u;
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Ranking key of (logit, expert): larger = ranked higher; ties go to the lower
// expert index.  0 is reserved for "already taken / no expert".
__device__ __forceinline__ uint64_t rank_key(float logit, int e) {
  return ((uint64_t)float_order_key(logit) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e);
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
  lo = __shfl_xor(lo, m, kWave);
  hi = __shfl_xor(hi, m, kWave);
  return ((uint64_t)hi << 32) | lo;
}

// Wave-wide max of a 64-bit key with a fixed butterfly.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    uint64_t o = shfl_xor_u64(v, m);
    v = o > v ? o : v;
  }
  return v;
}

// Wave-wide sum with a fixed butterfly (every lane gets the same bits).
__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

__device__ __forceinline__ int wave_sum_i32(int v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

// Inclusive prefix sum across the wave (lane order).
__device__ __forceinline__ int wave_incl_scan_i32(int v) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    int o = __shfl_up(v, d, kWave);
    if (lane >= d) v += o;
  }
  return v;
}

__host__ __device__ constexpr int ceil_div(int a, int b) { return (a + b - 1) / b; }

}  // namespace moe
