// stream.hip -- data movement of the streaming step: ring-slot copies of K/V
// frames and the copy (or zeroing) of the carried GLA state. HBM-bound copies,
// 16 bytes per lane, one grid-stride loop.
#include "device_common.h"
#include "hta_internal.h"

namespace hta {

namespace {

// dst[bh][dst_off + e] = src[bh][src_off + e] for e < n16*16 bytes, all bh.
__global__ __launch_bounds__(256) void copy_frames_kernel(const char* __restrict__ src,
                                                          char* __restrict__ dst, int BH,
                                                          long long src_bh, long long dst_bh,
                                                          long long n16) {
    const long long total = (long long)BH * n16;
    for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < total;
         i += (long long)gridDim.x * 256) {
        const long long bh = i / n16, e = i - bh * n16;
        *reinterpret_cast<u32x4*>(dst + bh * dst_bh + e * 16) =
            *reinterpret_cast<const u32x4*>(src + bh * src_bh + e * 16);
    }
}

__global__ __launch_bounds__(256) void fill_f32_kernel(float* __restrict__ dst,
                                                       const float* __restrict__ src, long long n) {
    for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n;
         i += (long long)gridDim.x * 256)
        dst[i] = src ? src[i] : 0.f;
}

// dst = a + b over n4 groups of 4 floats; each thread takes 4 groups 256 apart
// per pass, all loads issued before the stores (more bytes in flight per lane).
// dst = a + b over n4 float4 elements (dst may be a). Grid-stride rounds of 1024
// elements per block, eight loads in flight per thread; streaming (nontemporal)
// accesses, since nothing reads these arrays again soon.
__global__ __launch_bounds__(256) void add_f32_kernel(void* __restrict__ dst, int dst_bf16,
                                                      const float* a, const float* b, long long n4) {
    const long long step = (long long)gridDim.x * 1024;
    const f32x4* av = reinterpret_cast<const f32x4*>(a);
    const f32x4* bv = reinterpret_cast<const f32x4*>(b);
    for (long long base = (long long)blockIdx.x * 1024 + threadIdx.x; base < n4; base += step) {
        f32x4 x[4], y[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const long long i = base + 256 * u;
            if (i < n4) {
                x[u] = __builtin_nontemporal_load(av + i);
                y[u] = __builtin_nontemporal_load(bv + i);
            }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const long long i = base + 256 * u;
            if (i >= n4) break;
            const f32x4 r = f32x4{x[u][0] + y[u][0], x[u][1] + y[u][1], x[u][2] + y[u][2],
                                  x[u][3] + y[u][3]};
            if (dst_bf16) {
                bf16x4 o;
#pragma unroll
                for (int k = 0; k < 4; ++k) o[k] = f2bf(r[k]);
                __builtin_nontemporal_store(o, reinterpret_cast<bf16x4*>(dst) + i);
            } else {
                __builtin_nontemporal_store(r, reinterpret_cast<f32x4*>(dst) + i);
            }
        }
    }
}

unsigned grid_for(long long work) {
    long long g = (work + 255) / 256;
    if (g > 8192) g = 8192;
    return (unsigned)(g < 1 ? 1 : g);
}

}  // namespace

// Copies `elems` elements per (b,h) slice; byte offsets and strides are elems * elem_bytes.
hipError_t launch_copy_frames(const void* src, void* dst, int BH, long long src_bh,
                              long long dst_bh, long long src_off, long long dst_off,
                              long long elems, int elem_bytes, hipStream_t stream) {
    const long long bytes = elems * elem_bytes;
    if (BH == 0 || bytes == 0) return hipSuccess;
    if ((bytes & 15) || ((src_bh * elem_bytes) & 15) || ((dst_bh * elem_bytes) & 15) ||
        ((src_off * elem_bytes) & 15) || ((dst_off * elem_bytes) & 15))
        return hipErrorInvalidValue;
    const long long n16 = bytes / 16;
    hipLaunchKernelGGL(copy_frames_kernel, dim3(grid_for((long long)BH * n16)), dim3(256), 0, stream,
                       static_cast<const char*>(src) + src_off * elem_bytes,
                       static_cast<char*>(dst) + dst_off * elem_bytes, BH, src_bh * elem_bytes,
                       dst_bh * elem_bytes, n16);
    return hipGetLastError();
}

hipError_t launch_add_f32(void* dst, int dst_bf16, const float* a, const float* b, long long n,
                          hipStream_t stream) {
    if (n == 0) return hipSuccess;
    if (n & 3) return hipErrorInvalidValue;
    long long g = (n / 4 + 1023) / 1024;
    if (g > 4096) g = 4096;   // 16 workgroups per CU, then grid-stride
    hipLaunchKernelGGL(add_f32_kernel, dim3((unsigned)(g < 1 ? 1 : g)), dim3(256), 0, stream, dst,
                       dst_bf16, a, b, n / 4);
    return hipGetLastError();
}

hipError_t launch_fill_f32(float* dst, const float* src, long long n, hipStream_t stream) {
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(fill_f32_kernel, dim3(grid_for(n)), dim3(256), 0, stream, dst, src, n);
    return hipGetLastError();
}

}  // namespace hta
