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

template <typename T>
__global__ __launch_bounds__(256) void combine_rows(const T* __restrict__ y, const float* __restrict__ gates,
                                                   const uint8_t* __restrict__ kept, const T* __restrict__ shared,
                                                   const T* __restrict__ residual, T* __restrict__ out, int Tn, int H,
                                                   int k) {
  typedef typename Vec8<T>::type V;
  const int per_row = H / 8;
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (long)Tn * per_row) return;
  const int t = (int)(i / per_row);
  const long col = (long)(i % per_row) * 8;
  float acc[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) acc[q] = -0.0f;
  for (int j = 0; j < k; ++j) {
    const long r = (long)t * k + j;
    if (!kept[r]) continue;
    const float g = gates[r];
    const V v = *reinterpret_cast<const V*>(y + r * H + col);
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] = fmaf(g, (float)v[q], acc[q]);
  }
  if (shared) {
    const V v = *reinterpret_cast<const V*>(shared + (long)t * H + col);
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] += (float)v[q];
  }
  if (residual) {
    const V v = *reinterpret_cast<const V*>(residual + (long)t * H + col);
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] += (float)v[q];
  }
  V o;
#pragma unroll
  for (int q = 0; q < 8; ++q) o[q] = cvt_act<T>(acc[q]);
  *reinterpret_cast<V*>(out + (long)t * H + col) = o;
}

}  // namespace

hipError_t launch_combine(const moe_config& c, const void* y_route, const float* gates, const uint8_t* kept,
                          const void* shared_out, const void* residual, void* out, hipStream_t s) {
  const long n = (long)c.T * (c.H / 8);
  const dim3 grid((unsigned)((n + 255) / 256));
  if (c.act_dtype == MOE_F32) {
    combine_rows<float><<<grid, 256, 0, s>>>((const float*)y_route, gates, kept, (const float*)shared_out,
                                             (const float*)residual, (float*)out, c.T, c.H, c.k);
  } else {
    combine_rows<__bf16><<<grid, 256, 0, s>>>((const __bf16*)y_route, gates, kept, (const __bf16*)shared_out,
                                              (const __bf16*)residual, (__bf16*)out, c.T, c.H, c.k);
  }
  return hipGetLastError();
}

}  // namespace moe
