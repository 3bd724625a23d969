/*
 * hta_peaks.h -- C ABI of libhta_peaks: microbenchmarks of the ceilings the
 * rooflines of libhta are measured against on MI355X (gfx950), so that each
 * fraction can be stated against the published peak and against what the chip
 * delivers to a plain kernel:
 *   - an MFMA issue loop: bf16 matrix products on register operands with
 *     independent accumulators (no memory traffic in the loop);
 *   - a streaming copy through HBM;
 *   - the two on-chip paths the kernels' tiles take: direct global->LDS loads
 *     (global_load_lds_dwordx4) and LDS reads (ds_read_b128, ds_read_b64_tr_b16).
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

/*
 * hta_peak_lds_dma -- `blocks` workgroups of 4 waves; each wave issues `iters`
 * rounds of 8 direct global->LDS loads of 16 bytes per lane (1 KiB per load)
 * into a 16 KiB ring of its own, at most 16 loads in flight, and waits for all
 * of them at the end. pattern 0: each load reads 1 KiB of contiguous memory;
 * pattern 1: 32 rows of 32 bytes, 256 bytes apart (the shape of a 16-column
 * slice of a bf16 tile). The loads of wave w walk src + (w * iters * 64 KiB +
 * 8 KiB * i) mod window_bytes, so a window that fits in L2 measures the
 * L2->LDS path and a large one streams from HBM. window_bytes: a power of two,
 * >= 8192, all of it readable at src. Bytes loaded: blocks * 4 * iters * 8 *
 * 1024. Returns 0, or -1 for a NULL src, -2 for blocks or iters < 1, a bad
 * window or pattern, -10 for a src not 16-byte aligned, -8 if the launch fails.
 */
int hta_peak_lds_dma(const void* src, size_t window_bytes, int blocks, int iters, int pattern,
                     void* stream);

/*
 * hta_peak_lds_read -- `blocks` workgroups of 4 waves; each wave reads a
 * 64 KiB LDS buffer `iters` rounds of 8 loads: transposed == 0:
 * ds_read_b128 (16 bytes per lane), otherwise ds_read_b64_tr_b16 (8 bytes per
 * lane). One float per thread goes to sink[blocks * 256]. Bytes read:
 * blocks * 4 * iters * 8 * (transposed ? 512 : 1024). Returns 0, or -1 for a
 * NULL sink, -2 for blocks or iters < 1, -8 if the launch fails.
 */
int hta_peak_lds_read(int blocks, int iters, int transposed, float* sink, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* HTA_PEAKS_H */
