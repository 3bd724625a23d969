// peaks.hip -- the ceilings libhta's rooflines are set against, measured by
// plain kernels: an MFMA issue loop and a streaming HBM copy (include/hta_peaks.h).
#include <stdint.h>

#include "../../../include/hta_peaks.h"
#include "device_common.h"

namespace {

using hta::bf16;
using hta::bf16x8;
using hta::f32x16;
using hta::u32x4;

constexpr int kChains = 4;   // independent accumulators per wave

// Each wave: iters rounds of kChains independent v_mfma_f32_32x32x16_bf16 on
// register operands (distinct per chain, so no two chains compute the same
// values). Two waves per SIMD (2 workgroups of 4 waves per CU) hide the MFMA
// latency.
__global__ __launch_bounds__(256) void mfma_loop_kernel(int iters, float* sink) {
    const int t = threadIdx.x;
    bf16x8 a0, a1, b0, b1;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a0[i] = (bf16)(1e-3f * (float)((t + i) & 7));
        a1[i] = (bf16)(1e-3f * (float)((t + 2 * i + 1) & 7));
        b0[i] = (bf16)(1e-3f * (float)((t * 3 + i) & 7));
        b1[i] = (bf16)(1e-3f * (float)((t * 5 + i + 3) & 7));
    }
    f32x16 c0, c1, c2, c3;
#pragma unroll
    for (int r = 0; r < 16; ++r) c0[r] = c1[r] = c2[r] = c3[r] = 0.f;
    static_assert(kChains == 4, "four accumulators");
    for (int i = 0; i < iters; ++i) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b0, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b0, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b1, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b1, c3, 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
    sink[(size_t)blockIdx.x * 256 + t] = s;
}

// Grid-stride copy, four independent 16-byte loads in flight per thread.
__global__ __launch_bounds__(256) void hbm_copy_kernel(const u32x4* __restrict__ src,
                                                       u32x4* __restrict__ dst, long long n16) {
    const long long stride = (long long)gridDim.x * 256 * 4;
    for (long long i = (long long)blockIdx.x * 256 * 4 + threadIdx.x; i < n16; i += stride) {
        u32x4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = src[i + u * 256];
#pragma unroll
        for (int u = 0; u < 4; ++u) dst[i + u * 256] = v[u];
    }
}

}  // namespace

extern "C" {

int hta_peak_mfma_chains(void) { return kChains; }

int hta_peak_mfma(int blocks, int iters, float* sink, void* stream) {
    if (!sink) return -1;
    if (blocks < 1 || iters < 1) return -2;
    mfma_loop_kernel<<<blocks, 256, 0, static_cast<hipStream_t>(stream)>>>(iters, sink);
    return hipGetLastError() == hipSuccess ? 0 : -8;
}

int hta_peak_copy(const void* src, void* dst, size_t bytes, void* stream) {
    if (!src || !dst) return -1;
    if (bytes == 0 || bytes % 16384) return -2;
    const uintptr_t s = reinterpret_cast<uintptr_t>(src), d = reinterpret_cast<uintptr_t>(dst);
    if ((s | d) & 15) return -10;
    if (s < d + bytes && d < s + bytes) return -9;
    // n16 is a multiple of 1024 and every round of a block starts at a multiple
    // of 1024: when i = base + tid < n16, all of i + u * 256 (u < 4) are too.
    const long long n16 = (long long)(bytes / 16);
    const long long want = n16 / 1024;
    const int blocks = (int)(want < 8192 ? want : 8192);
    hbm_copy_kernel<<<blocks, 256, 0, static_cast<hipStream_t>(stream)>>>(
        static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), n16);
    return hipGetLastError() == hipSuccess ? 0 : -8;
}

}  // extern "C"
