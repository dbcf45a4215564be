// Measured ceilings for the roofline: HBM copy / read streams and bf16 MFMA issue.
// Declared in include/moe_ceiling.h; built into libmoe_ceiling.so, separate from
// the layer's library.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_ceiling.h"

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kUnroll = 8;            // 16-byte vectors in flight per lane
constexpr int kBlocksPerCU = 8;       // 32 resident waves per CU
constexpr size_t kPer = (size_t)kThreads * kUnroll;  // vectors per workgroup pass

// Streaming copy: each workgroup pass moves kPer contiguous 16-byte vectors, all kUnroll
// loads of a lane issued before its first store; load j of the wave covers 1 KB of
// consecutive bytes.  Non-temporal, so the stream does not sit in the caches.
__global__ __launch_bounds__(kThreads) void copy16(const u32x4* __restrict__ src, u32x4* __restrict__ dst, size_t n) {
  for (size_t base = (size_t)blockIdx.x * kPer; base < n; base += (size_t)gridDim.x * kPer) {
    u32x4 v[kUnroll];
    if (base + kPer <= n) {
#pragma unroll
      for (int j = 0; j < kUnroll; ++j) v[j] = __builtin_nontemporal_load(src + base + j * kThreads + threadIdx.x);
#pragma unroll
      for (int j = 0; j < kUnroll; ++j) __builtin_nontemporal_store(v[j], dst + base + j * kThreads + threadIdx.x);
    } else {
      for (int j = 0; j < kUnroll; ++j) {
        const size_t i = base + j * kThreads + threadIdx.x;
        if (i < n) dst[i] = src[i];
      }
    }
  }
}

// Streaming read: the same pattern, folding the data into one word so the loads stay.
__global__ __launch_bounds__(kThreads) void read16(const u32x4* __restrict__ src, size_t n, float* __restrict__ sink) {
  unsigned x = 0;
  for (size_t base = (size_t)blockIdx.x * kPer; base < n; base += (size_t)gridDim.x * kPer) {
    u32x4 v[kUnroll];
    if (base + kPer <= n) {
#pragma unroll
      for (int j = 0; j < kUnroll; ++j) v[j] = __builtin_nontemporal_load(src + base + j * kThreads + threadIdx.x);
    } else {
#pragma unroll
      for (int j = 0; j < kUnroll; ++j) {
        const size_t i = base + j * kThreads + threadIdx.x;
        v[j] = i < n ? src[i] : u32x4{};
      }
    }
#pragma unroll
    for (int j = 0; j < kUnroll; ++j) x ^= v[j][0] ^ v[j][1] ^ v[j][2] ^ v[j][3];
  }
  if (x == 0x9e3779b9u) sink[blockIdx.x % 4096] = (float)x;
}

// Workgroups for n vectors: one pass each where possible, at most kBlocksPerCU per CU.
unsigned stream_grid(size_t n) {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    cus = 256;
  const size_t passes = (n + kPer - 1) / kPer;
  const size_t cap = (size_t)cus * kBlocksPerCU;
  return (unsigned)(passes < cap ? passes : cap);
}

template <int WPE>
__global__ __launch_bounds__(256 * WPE) __attribute__((amdgpu_waves_per_eu(WPE, WPE))) void mfma_loop(int iters,
                                                                                                    float* sink) {
  __shared__ char pin[100000];  // one workgroup per CU
  if (iters < 0) pin[threadIdx.x] = 1;
  bf16x8 a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(threadIdx.x * 0.001f + i);
    b[i] = (__bf16)(i * 0.5f);
  }
  f32x16 acc[8];
  for (int j = 0; j < 8; ++j) acc[j] = f32x16{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
  }
  float s = 0.f;
  for (int j = 0; j < 8; ++j)
    for (int r = 0; r < 16; ++r) s += acc[j][r];
  if (s == 1234.5f) sink[threadIdx.x] = s + pin[threadIdx.x];
}

int32_t status(hipError_t e) { return e == hipSuccess ? 0 : 6; }

}  // namespace

extern "C" {

int32_t moe_ceiling_copy(const void* src, void* dst, size_t bytes, void* stream) {
  if (!src || !dst || bytes == 0 || bytes % 16 || ((uintptr_t)src | (uintptr_t)dst) % 16) return 1;
  copy16<<<stream_grid(bytes / 16), kThreads, 0, (hipStream_t)stream>>>((const u32x4*)src, (u32x4*)dst, bytes / 16);
  return status(hipGetLastError());
}

int32_t moe_ceiling_read(const void* src, size_t bytes, float* sink, void* stream) {
  if (!src || !sink || bytes == 0 || bytes % 16 || (uintptr_t)src % 16) return 1;
  read16<<<stream_grid(bytes / 16), kThreads, 0, (hipStream_t)stream>>>((const u32x4*)src, bytes / 16, sink);
  return status(hipGetLastError());
}

int32_t moe_ceiling_clock_rates(int32_t* wall_khz, int32_t* peak_khz) {
  if (!wall_khz || !peak_khz) return 1;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(wall_khz, hipDeviceAttributeWallClockRate, dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(peak_khz, hipDeviceAttributeClockRate, dev);
  return status(e);
}

int32_t moe_ceiling_mfma_bf16(int32_t iters, int32_t waves_per_simd, float* sink, void* stream) {
  if (!sink || iters <= 0 || (waves_per_simd != 1 && waves_per_simd != 2)) return 1;
  if (waves_per_simd == 1)
    mfma_loop<1><<<256, 256, 0, (hipStream_t)stream>>>(iters, sink);
  else
    mfma_loop<2><<<256, 512, 0, (hipStream_t)stream>>>(iters, sink);
  return status(hipGetLastError());
}

}  // extern "C"
