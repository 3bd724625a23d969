// peaks.hip -- the ceilings libhta's rooflines are set against, measured by
// plain kernels: an MFMA issue loop, a streaming HBM copy, direct global->LDS
// loads and LDS reads (include/hta_peaks.h).
#include <stdint.h>

#include "../../../include/hta_peaks.h"
#include "device_common.h"

namespace {

using hta::bf16;
using hta::bf16x4;
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

// s_waitcnt on the vector-memory counter only (gfx9 encoding): everything but
// the newest N loads of this wave has completed.
template <int N>
__device__ __forceinline__ void wait_vm() {
    __builtin_amdgcn_s_waitcnt((N & 0xF) | (((N >> 4) & 0x3) << 14) | (0x7 << 4) | (0xF << 8));
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    typedef __attribute__((address_space(3))) const char lds_char;
    return (uint32_t)(uintptr_t)(lds_char*)p;
}

// 16 bytes per lane from sbase + voff into LDS at lds + 16 * lane.
__device__ __forceinline__ void load_lds16(uint32_t voff, const void* sbase, uint32_t lds) {
    const uint64_t b = (uint64_t)(uintptr_t)sbase;
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));
    const uint64_t sb = ((uint64_t)hi << 32) | (uint64_t)lo;
    const uint32_t ls = (uint32_t)__builtin_amdgcn_readfirstlane((int)lds);
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" : : "s"(ls), "v"(voff), "s"(sb) : "m0");
}

// Each wave: iters rounds of 8 loads of 1 KiB into its 16 KiB ring slot by slot;
// after each round at most 8 more may stay in flight. Offsets are multiples of
// 8 KiB below the window, and a load spans at most 8 KiB.
template <int PATTERN>
__global__ __launch_bounds__(256) void lds_dma_kernel(const char* src, unsigned long long mask, int iters) {
    extern __shared__ __attribute__((aligned(1024))) char ring[];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint32_t base = lds_addr(ring) + (uint32_t)wave * 16384u;
    const unsigned long long gw = (unsigned long long)blockIdx.x * 4 + wave;
    const unsigned long long start = gw * (unsigned long long)iters * 65536ull;
    const uint32_t voff = PATTERN == 0 ? (uint32_t)lane * 16u
                                       : (uint32_t)((lane >> 1) * 256 + (lane & 1) * 16);
    int slot = 0;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const unsigned long long o = (start + (unsigned long long)(it * 8 + u) * 8192ull) & mask;
            load_lds16(voff, src + o, base + (uint32_t)slot * 1024u);
            slot = (slot + 1) & 15;
        }
        wait_vm<8>();
    }
    wait_vm<0>();
}

// Each wave reads its part of a 64 KiB LDS buffer, 8 loads a round, and keeps a
// sum so the loads cannot be removed.
template <bool TR>
__global__ __launch_bounds__(256) void lds_read_kernel(int iters, float* sink) {
    __shared__ __attribute__((aligned(16))) float buf[16384];
    if (TR) {   // read as bf16: every 16-bit half a finite bf16
        bf16* hb = reinterpret_cast<bf16*>(buf);
        for (int i = threadIdx.x; i < 32768; i += 256) hb[i] = (bf16)((float)(i & 255) * 1e-3f);
    } else {
        for (int i = threadIdx.x; i < 16384; i += 256) buf[i] = (float)(i & 255) * 1e-3f;
    }
    __syncthreads();
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    float acc = 0.f;
    if (!TR) {
        typedef float f4 __attribute__((ext_vector_type(4)));
        const f4* b4 = reinterpret_cast<const f4*>(buf);
        int idx = (lane + wave * 64) & 4095;   // 16 bytes per lane, contiguous per wave
        f4 s = {0.f, 0.f, 0.f, 0.f};
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int u = 0; u < 8; ++u) s += b4[(idx + u * 256) & 4095];
            idx = (idx + 16) & 4095;
        }
        acc = s[0] + s[1] + s[2] + s[3];
    } else {
        typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
        const char* cb = reinterpret_cast<const char*>(buf);
        int off = (lane * 8 + wave * 512) & 65535;   // 8 bytes per lane
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const bf16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                    (lds_bf16x4*)(cb + ((off + u * 4096) & 65535)));
                acc += (float)v[0] + (float)v[3];
            }
            off = (off + 64) & 65535;
        }
    }
    sink[(size_t)blockIdx.x * 256 + threadIdx.x] = acc;
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

int hta_peak_lds_dma(const void* src, size_t window_bytes, int blocks, int iters, int pattern,
                     void* stream) {
    if (!src) return -1;
    if (blocks < 1 || iters < 1 || (pattern != 0 && pattern != 1)) return -2;
    if (window_bytes < 8192 || (window_bytes & (window_bytes - 1))) return -2;
    if (reinterpret_cast<uintptr_t>(src) & 15) return -10;
    const unsigned long long mask = (unsigned long long)window_bytes - 1;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    constexpr int kLds = 65536;
    if (pattern == 0) {
        if (hipFuncSetAttribute(reinterpret_cast<const void*>(lds_dma_kernel<0>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, kLds) != hipSuccess)
            return -8;
        lds_dma_kernel<0><<<blocks, 256, kLds, st>>>(static_cast<const char*>(src), mask, iters);
    } else {
        if (hipFuncSetAttribute(reinterpret_cast<const void*>(lds_dma_kernel<1>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, kLds) != hipSuccess)
            return -8;
        lds_dma_kernel<1><<<blocks, 256, kLds, st>>>(static_cast<const char*>(src), mask, iters);
    }
    return hipGetLastError() == hipSuccess ? 0 : -8;
}

int hta_peak_lds_read(int blocks, int iters, int transposed, float* sink, void* stream) {
    if (!sink) return -1;
    if (blocks < 1 || iters < 1) return -2;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    if (transposed)
        lds_read_kernel<true><<<blocks, 256, 0, st>>>(iters, sink);
    else
        lds_read_kernel<false><<<blocks, 256, 0, st>>>(iters, sink);
    return hipGetLastError() == hipSuccess ? 0 : -8;
}

}  // extern "C"
