/*
 * svdq_peaks.h -- measurement kernels of libsvdq: the second denominators of the roofline
 * fractions the benchmark reports next to the published MI355X peaks.  They compute nothing
 * of the method; a benchmark times them with events on `stream`.
 *
 * svdq_peak_mfma: one launch of a kernel that keeps every SIMD of the GPU issuing
 *   independent back-to-back MFMAs of one kind (two waves per SIMD, four accumulator chains
 *   per wave, `iters` instructions per chain), with operands held in registers.  kind:
 *     0  v_mfma_scale_f32_32x32x64_f8f6f4, FP6 E2M3 operands (the packed INT4 GEMM's)
 *     1  v_mfma_i32_32x32x32_i8 (the nibble-operand INT4 GEMM's)
 *     2  v_mfma_f32_32x32x16_bf16
 *     3  v_mfma_f32_32x32x8_bf16 (the packed GEMM's scale-product instruction)
 *     4  v_mfma_f32_32x32x16_f16 (the NVFP4 GEMM's)
 *     5  v_mfma_scale_f32_32x32x64_f8f6f4, FP4 E2M1 operands
 *   `out` is device memory of at least one float (written, so the work is not optimised
 *   away); *ops (host) receives the operations one launch performs (2 m n k per MFMA, a
 *   multiply-add counted as two).  iters in [1, 1 << 20]; SVDQ_ERR_INVALID_ARG otherwise.
 * svdq_peak_copy: dst[0, bytes) = src[0, bytes), 16-byte loads and stores, a grid-stride
 *   loop over the whole GPU; src and dst device memory, 16-byte aligned, not overlapping,
 *   bytes a positive multiple of 16.  It moves 2 * bytes through HBM.
 * svdq_peak_read: loads src[0, bytes) once (16-byte non-temporal loads, a grid-stride loop
 *   with four loads per thread in flight); `out` is device memory of at least 4 bytes,
 *   written only with a value the data cannot produce (so in practice never).  bytes a
 *   positive multiple of 16, src 16-byte aligned.  It moves `bytes` through HBM.
 * All check the device like every other entry point and enqueue on `stream`.
 */
#ifndef SVDQ_PEAKS_H
#define SVDQ_PEAKS_H

#include <stdint.h>

#include "svdq.h"

#ifdef __cplusplus
extern "C" {
#endif

svdq_status svdq_peak_mfma(int32_t kind, int32_t iters, float* out, int64_t* ops,
                           svdq_stream_t stream);
svdq_status svdq_peak_copy(const void* src, void* dst, int64_t bytes, svdq_stream_t stream);
svdq_status svdq_peak_read(const void* src, int64_t bytes, void* out, svdq_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SVDQ_PEAKS_H */
