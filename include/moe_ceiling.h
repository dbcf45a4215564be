/*
 * moe_ceiling.h -- C ABI of libmoe_ceiling.so: measured hardware ceilings that the
 * MoE layer's kernels are compared with (not part of the layer).
 *
 * All calls enqueue one kernel on `stream` (a hipStream_t, NULL = null stream) and
 * return 0 on success, 1 for a bad argument (NULL pointer, misaligned pointer,
 * non-positive size), 6 if the launch failed.  The caller owns every buffer.
 */
#ifndef MOE_CEILING_H_
#define MOE_CEILING_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* dst[0:bytes) = src[0:bytes): a streaming copy (8 non-temporal 16-byte loads in flight
 * per lane, then their stores; up to 8 workgroups of 256 lanes per CU).  bytes % 16 == 0,
 * both pointers 16-byte aligned.  Moves 2 * bytes through HBM when the buffers exceed the
 * caches; also the known-size reference for traffic counters. */
int32_t moe_ceiling_copy(const void* src, void* dst, size_t bytes, void* stream);

/* Reads src[0:bytes) as a stream (the copy's access pattern, no stores) and writes one float
 * per workgroup to sink[0:4096) only for a sentinel value, so the reads cannot be elided.
 * bytes % 16 == 0, src 16-byte aligned. */
int32_t moe_ceiling_read(const void* src, size_t bytes, float* sink, void* stream);

/* Every SIMD of every CU issues iters x 8 independent v_mfma_f32_32x32x16_bf16 from
 * registers (waves_per_simd 1 or 2); writes nothing unless the result is a
 * sentinel (sink has 1024 floats).  FLOP = 256 CUs x 4 SIMDs x waves_per_simd x
 * iters x 8 x 32768. */
int32_t moe_ceiling_mfma_bf16(int32_t iters, int32_t waves_per_simd, float* sink, void* stream);

/* Host only: the current device's wall-clock counter rate (the rate of HIP wall_clock64)
 * and its peak shader clock, both in kHz (hipDeviceGetAttribute).  Returns 1 for a NULL
 * pointer, 6 if the query fails. */
int32_t moe_ceiling_clock_rates(int32_t* wall_khz, int32_t* peak_khz);

#ifdef __cplusplus
}
#endif

#endif /* MOE_CEILING_H_ */
