/*
 * pic_peaks.h -- C ABI of libpicpeaks.so: machine peaks measured on the GPU,
 * the denominators a benchmark reports beside the vendor figures (MI355X:
 * 8 TB/s HBM3E, 2.5 PFLOP/s dense bf16 MFMA).  Not part of the attention
 * library; every function allocates its own device memory, runs on a stream
 * of its own, synchronises it and frees everything before returning.
 * Return value: 0 on success, -1 for a bad argument, otherwise the failing
 * hipError_t.  The result is 0 on failure.
 */
#ifndef PIC_PEAKS_H
#define PIC_PEAKS_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Streaming read of `bytes` (>= 1 MiB) of device memory, `reps` timed passes
 * after one untimed pass, for each of six kernel shapes (4 or 8 16-byte loads
 * in flight per thread, plain or non-temporal, 8 or 16 workgroups per CU):
 * the best achieved GB/s (1e9 bytes per second). */
int pic_peak_hbm_read(size_t bytes, int reps, double *gbytes_per_s);

/* Dense bf16 MFMA issue rate from register-resident operands, 8 waves per
 * SIMD: shape 16 = v_mfma_f32_16x16x32_bf16 (4 chains per wave), shape 32 =
 * v_mfma_f32_32x32x16_bf16 (2 chains per wave); `iters` loop trips per wave.
 * Result in TFLOP/s (2 m n k flops per MFMA). */
int pic_peak_mfma_bf16(int shape, int iters, double *tflops);

/* v_exp_f32 issue rate: 8 independent dependent chains per lane, `iters`
 * trips.  Result in 1e9 exponentials per second over the whole GPU. */
int pic_peak_exp2(int iters, double *gexp_per_s);

#ifdef __cplusplus
}
#endif

#endif /* PIC_PEAKS_H */
