/* Roofline probes exported by libgdr.so next to the forward (gdr.h).
 *
 * Neither computes anything of the delta rule. They measure, on the GPU the
 * library runs on, the two ceilings the forward is reported against: HBM
 * bandwidth (a streaming copy) and dense bf16 matrix-core throughput (a loop
 * of independent v_mfma_f32_16x16x32_bf16). A benchmark times them with its
 * own events on `stream`.
 *
 * Ownership: the caller owns every buffer; nothing is allocated. Calls are
 * asynchronous on `stream` (a hipStream_t, NULL for the default stream).
 * Return value: 0 on success, 1 for an invalid argument (nothing enqueued),
 * 2 when the launch failed.
 */
#ifndef GDR_PEAKS_H
#define GDR_PEAKS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Copies `bytes` (a multiple of 16) from device buffer src to device buffer
 * dst, both 16-byte aligned and not overlapping, with `blocks` workgroups of
 * 256 lanes reading and writing 16 bytes per lane per access (non-temporal).
 * Moves 2 * bytes through HBM. */
int gdr_peak_copy(const void* src, void* dst, size_t bytes, int32_t blocks, void* stream);

/* `blocks` workgroups of four wavefronts; each wavefront issues iters x 8
 * independent bf16 16x16x32 matrix-core products and writes one float per
 * lane to out (device buffer of blocks * 256 floats). */
int gdr_peak_mfma(float* out, int32_t blocks, int32_t iters, void* stream);

/* Floating-point operations (2 per multiply-add) one gdr_peak_mfma call with
 * these arguments performs. */
double gdr_peak_mfma_flops(int32_t blocks, int32_t iters);

#ifdef __cplusplus
}
#endif

#endif /* GDR_PEAKS_H */
