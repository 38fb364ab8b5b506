/*
 * qlin_peaks -- the two reference kernels that measure what one MI355X
 * actually delivers, so that the matmul kernels' rates can be reported as a
 * fraction of an achieved peak as well as of the published one.  Measurement
 * utilities, not part of the matmul interface (include/qlin.h).
 *
 * Both enqueue one kernel on `stream` and return the HIP error code (0 = ok).
 */
#ifndef QLIN_PEAKS_H
#define QLIN_PEAKS_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Streaming read: every 16-byte word of src[0, bytes) is loaded once
 * (bytes a multiple of 16 and at least 16 * qlin_peak_read_groups(), src
 * 16-byte aligned; else hipErrorInvalidValue) and folded into one uint32 per
 * work-group, written to sink[0 .. qlin_peak_read_groups() - 1] (so the loads
 * cannot be removed).  Each of the 16384 work-groups of 256 threads reads one
 * contiguous chunk with 16 loads in flight per thread. */
int qlin_peak_stream_read(const void* src, int64_t bytes, uint32_t* sink, hipStream_t stream);
int64_t qlin_peak_read_groups(void);

/* Matrix-core loop: `iters` rounds of 8 independent
 * v_mfma_f32_32x32x16_f16 per wave, no memory traffic in the loop; each wave
 * writes one float of its accumulators to sink[wave] (sink holds
 * qlin_peak_mfma_waves() floats).  Work = waves * iters * 8 * 32768 flop. */
int qlin_peak_mfma(int32_t iters, float* sink, hipStream_t stream);
int64_t qlin_peak_mfma_waves(void);

#ifdef __cplusplus
}
#endif

#endif /* QLIN_PEAKS_H */
