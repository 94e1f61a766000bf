/*
 * pisa_peaks.h -- microbenchmarks of the MI355X units that bound the PISA
 * selection path, so that a benchmark can time them in the same run as the
 * kernels it reports (libpisa_peaks.so; not part of the selection library).
 *
 * The leaf-level scoring of "Block Sparse Attention with Log-Linear
 * Complexity" (section 3.2 eq 21, section 3.3 eq 23-24) is a bf16 product
 * followed by one exponential per logit for the exact log-sum-exp, so its
 * floor is set by the matrix cores, the transcendental unit, or both at once.
 * Each call queues one kernel on `stream` (a hipStream_t, NULL = default) and
 * returns 0, or -1 for bad arguments, -4 for a launch error. Nothing is
 * allocated; `out` is a device buffer of at least blocks * 256 floats that
 * receives one value per thread (so the loops cannot be removed).
 *
 *   pisa_peak_exp:  per thread, 8 independent chains x <- 2^(-x), iters
 *                   times: blocks * 256 * iters * 8 v_exp_f32 lane results.
 *   pisa_peak_mfma: per wave, 8 independent accumulators, iters times each:
 *                   blocks * 4 * iters * 8 MFMA 16x16x32 bf16 (16,384 flops each).
 *   pisa_peak_mix:  per wave and iteration, 8 MFMA 16x16x32 bf16 and 8
 *                   v_exp_f32 on every lane (the 1:1 mix of MFMA and wave-wide
 *                   exponentials of the leaf scoring of a 16 x 64 logit tile).
 *   pisa_peak_copy: dst[i] = src[i] for bytes (a multiple of 16, 16-byte
 *                   aligned pointers) with 16-byte loads and stores.
 *   pisa_peak_read: reads src[0, bytes) once with 16-byte loads (bytes a
 *                   multiple of 16, src 16-byte aligned); out holds 2048 * 256
 *                   floats.
 *   pisa_peak_gather: every wave reads rows_per_wave (a multiple of 8, >= 8)
 *                   rows of 1 KiB at hashed positions among the bytes / 1024
 *                   whole rows of src (16-byte aligned, bytes >= 1024 and
 *                   below 2^42): blocks * 4 * rows_per_wave KiB read, the
 *                   access pattern of the routers' per-entry query gathers
 *                   (G_Q = 4 heads of d = 128 bf16 per entry).
 */
#ifndef PISA_PEAKS_H
#define PISA_PEAKS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int pisa_peak_exp(float* out, int32_t blocks, int32_t iters, void* stream);
int pisa_peak_mfma(float* out, int32_t blocks, int32_t iters, void* stream);
int pisa_peak_mix(float* out, int32_t blocks, int32_t iters, void* stream);
int pisa_peak_copy(const void* src, void* dst, size_t bytes, void* stream);
int pisa_peak_read(const void* src, size_t bytes, float* out, void* stream);
int pisa_peak_gather(const void* src, size_t bytes, float* out, int32_t blocks, int32_t rows_per_wave,
                     uint32_t seed, void* stream);

#ifdef __cplusplus
}
#endif

#endif
