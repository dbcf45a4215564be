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

constexpr int kBlocks = 4096;
constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void copy16(const u32x4* __restrict__ src, u32x4* __restrict__ dst, size_t n) {
  for (size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += (size_t)gridDim.x * kThreads) dst[i] = src[i];
}

__global__ __launch_bounds__(kThreads) void read16(const u32x4* __restrict__ src, size_t n, float* __restrict__ sink) {
  unsigned x = 0;
  for (size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += (size_t)gridDim.x * kThreads) {
    const u32x4 v = src[i];
    x ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  if (x == 0x9e3779b9u) sink[blockIdx.x % 4096] = (float)x;
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
  copy16<<<kBlocks, kThreads, 0, (hipStream_t)stream>>>((const u32x4*)src, (u32x4*)dst, bytes / 16);
  return status(hipGetLastError());
}

int32_t moe_ceiling_read(const void* src, size_t bytes, float* sink, void* stream) {
  if (!src || !sink || bytes == 0 || bytes % 16 || (uintptr_t)src % 16) return 1;
  read16<<<kBlocks, kThreads, 0, (hipStream_t)stream>>>((const u32x4*)src, bytes / 16, sink);
  return status(hipGetLastError());
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
