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

// LDS byte address of a shared-memory array (its address-space cast folds to a constant)
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)((__attribute__((address_space(3))) const void*)p);
}

// One global -> LDS copy (buffer_load_dwordx4 ... lds): lane L's 16 bytes at buffer offset
// voff + soff land at LDS byte address m0 + 16 L.  Written as inline assembly, so that the
// only waits for it are the kernel's own: the compiler's wait-count pass does not tell
// apart the LDS arrays the builtin form writes once several stages of copies are in
// flight, and makes every LDS read wait for all of them.  The copy reads M0 one wait
// state after the scalar write (s_nop 0).
__device__ __forceinline__ void lds_copy16(__amdgpu_buffer_rsrc_t r, uint32_t m0, uint32_t voff, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(m0), "v"(voff), "s"(r), "s"(soff)
               : "m0");
}

// Workgroup barrier without a memory fence: the caller has already waited for what the
// other waves need (__syncthreads() would also wait for every LDS copy in flight, which
// its workgroup fence counts as LDS writes).  The memory clobber keeps the compiler from
// moving memory operations across it.
__device__ __forceinline__ void bare_barrier() { asm volatile("s_barrier" ::: "memory"); }

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

// Lanes of this wave holding the same key (0 .. 2^KB - 1) as this lane, from KB ballots.
template <int KB = 9>
__device__ __forceinline__ uint64_t peer_mask(int key) {
  uint64_t peers = __ballot(1);
#pragma unroll
  for (int b = 0; b < KB; ++b) {
    const bool bit = (key >> b) & 1;
    const uint64_t bal = __ballot(bit);
    peers &= bit ? bal : ~bal;
  }
  return peers;
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

// Cross-lane moves inside rows of 16 lanes (DPP): swap neighbours (lane ^ 1), swap
// pairs (lane ^ 2), reverse each 8-lane half row, reverse the 16-lane row.  Applied
// in that order, each step joins two groups that already agree, so after step s every
// lane holds the reduction of its aligned group of 2^(s+1) lanes.
enum : int { kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140 };

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  return ((uint64_t)dpp_u32<CTRL>((uint32_t)(v >> 32)) << 32) | dpp_u32<CTRL>((uint32_t)v);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __uint_as_float(dpp_u32<CTRL>(__float_as_uint(v)));
}

// Max of a 64-bit key over each aligned group of L lanes (L = 8, 16, 32 or 64); every
// lane of a group gets the group's max.  Max is exact, so the step order cannot
// change the result.  A group's lanes must all be active together.
__device__ __forceinline__ uint64_t group_max_u64(uint64_t v, int L) {
  uint64_t o;
  o = dpp_u64<kDppXor1>(v);
  v = o > v ? o : v;
  o = dpp_u64<kDppXor2>(v);
  v = o > v ? o : v;
  o = dpp_u64<kDppHalfMirror>(v);
  v = o > v ? o : v;
  if (L > 8) {
    o = dpp_u64<kDppMirror>(v);
    v = o > v ? o : v;
  }
  if (L > 16) {
    o = shfl_xor_u64(v, 16);
    v = o > v ? o : v;
  }
  if (L > 32) {
    o = shfl_xor_u64(v, 32);
    v = o > v ? o : v;
  }
  return v;
}

// Sum over each aligned group of L lanes with a fixed pairing order; the two lanes of
// a pair add the same two values, so every lane of the group gets the same bits.
__device__ __forceinline__ float group_sum_f32(float v, int L) {
  v += dpp_f32<kDppXor1>(v);
  v += dpp_f32<kDppXor2>(v);
  v += dpp_f32<kDppHalfMirror>(v);
  if (L > 8) v += dpp_f32<kDppMirror>(v);
  if (L > 16) v += __shfl_xor(v, 16, kWave);
  if (L > 32) v += __shfl_xor(v, 32, kWave);
  return v;
}

// Lanes per token for the top-k: the fewest of 8, 16, 32 that hold N experts at up to
// kTopkPerLane each (N <= 64: 8, N <= 128: 16, N <= 256: 32), so that a wave ranks 8, 4 or
// 2 tokens at once.
constexpr int kTopkPerLane = 8;
__host__ __device__ inline int topk_lanes(int N) { return N <= 64 ? 8 : (N <= 128 ? 16 : 32); }

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

// Word 3 of a buffer resource for raw (untyped, stride 0) buffer loads on gfx9-family
// parts.  A load whose byte offset is at or beyond the resource's size returns zeros
// and touches no memory; a store there writes nothing.  kBufferOutOfRange is such an
// offset for every resource under 2 GiB, with room to add a few 16-byte pieces to it
// without wrapping around 2^32.
constexpr int kRawBufferFlags = 0x00020000;
constexpr uint32_t kBufferOutOfRange = 0x80000000u;

}  // namespace moe
