/*
 * hta_peaks.h -- C ABI of libhta_peaks: microbenchmarks of the two ceilings the
 * rooflines of libhta are measured against on MI355X (gfx950), so that each
 * fraction can be stated against the published peak and against what the chip
 * delivers to a plain kernel:
 *   - an MFMA issue loop: bf16 matrix products on register operands with
 *     independent accumulators (no memory traffic in the loop);
 *   - a streaming copy through HBM.
 * The timing itself is the caller's (HIP events on `stream` around the call).
 * All pointers are device pointers owned by the caller; calls are asynchronous
 * on `stream` (a hipStream_t as void*, NULL = the null stream). Every argument
 * is checked before anything is enqueued; a non-zero return enqueues nothing.
 */
#ifndef HTA_PEAKS_H
#define HTA_PEAKS_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * hta_peak_mfma -- `blocks` workgroups of 4 waves; each wave issues `iters`
 * rounds of hta_peak_mfma_chains() independent v_mfma_f32_32x32x16_bf16
 * (32768 FLOP per wave-instruction). Total work: blocks * 4 * iters * chains *
 * 32768 FLOP. One float per thread (the sum of its accumulators) goes to
 * sink[blocks * 256], so the loop cannot be removed. Returns 0, or -1 for a
 * NULL sink, -2 for blocks or iters < 1, -8 if the launch fails.
 */
int hta_peak_mfma(int blocks, int iters, float* sink, void* stream);
int hta_peak_mfma_chains(void);

/*
 * hta_peak_copy -- dst[0 .. bytes) = src[0 .. bytes): 16-byte loads and stores,
 * each element read and written once (HBM traffic 2 * bytes). bytes a
 * multiple of 16384 (-2 otherwise), src and dst 16-byte aligned (-10) and not
 * overlapping (-9). Returns 0, or -1 for NULL pointers, -8 if the launch fails.
 */
int hta_peak_copy(const void* src, void* dst, size_t bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* HTA_PEAKS_H */
