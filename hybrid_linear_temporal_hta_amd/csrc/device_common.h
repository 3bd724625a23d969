// device_common.h -- small device helpers shared by the libhta kernels (gfx950).
//
// bf16 storage, fp32 math. MFMA fragment conventions used throughout (wave64):
//   v_mfma_f32_32x32x16_bf16  D[32x32] += A[32x16] * B[16x32]
//     A: lane l holds A[m = l%32][k = 8*(l/32) + j], j = 0..7
//     B: lane l holds B[k = 8*(l/32) + j][n = l%32], j = 0..7
//     D: lane l holds D[m = 8*(i/4) + 4*(l/32) + i%4][n = l%32] in element i (0..15)
//   v_mfma_f32_16x16x32_bf16  D[16x16] += A[16x32] * B[32x16]
//     A: lane l holds A[m = l%16][k = 8*(l/16) + j]
//     B: lane l holds B[k = 8*(l/16) + j][n = l%16]
//     D: lane l holds D[m = 4*(l/16) + i][n = l%16] in element i (0..3)
// A contraction index may be permuted freely as long as A and B agree on it;
// the kernels use that to feed a D fragment back as a B fragment without a
// trip through LDS.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hta {

typedef __bf16 bf16;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16;
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma32h(f16x8 a, f16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma16h(f16x8 a, f16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float bf2f(bf16 x) { return (float)x; }
__device__ __forceinline__ bf16 f2bf(float x) { return (bf16)x; }  // round to nearest even

__device__ __forceinline__ bf16x8 cat(bf16x4 lo, bf16x4 hi) {
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ f16x8 cat(f16x4 lo, f16x4 hi) {
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Two bf16 in a dword -> two fp16 in a dword (round to nearest even; exact for
// |x| in the fp16 normal range, which covers the bf16 values it is used on).
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w) {
    const float lo = __uint_as_float(w << 16);
    const float hi = __uint_as_float(w & 0xffff0000u);
    const f16 a = (f16)lo, b = (f16)hi;
    return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

__device__ __forceinline__ u32x4 bf16x8_to_f16x8(u32x4 w) {
    return u32x4{bf16x2_to_f16x2(w[0]), bf16x2_to_f16x2(w[1]), bf16x2_to_f16x2(w[2]),
                 bf16x2_to_f16x2(w[3])};
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// acc + a.x + a.y for a pair of bf16 values (one v_dot2_f32_bf16 with ones).
__device__ __forceinline__ float add_pair(bf16x2 a, float acc) {
    const bf16x2 one = {(bf16)1.0f, (bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(a, one, acc, false);
}

// Combine lane l with lane l ^ 32 (the two halves of a wave) on the VALU:
// v_permlane32_swap with both operands x returns (x[lo], x[lo]) and (x[hi], x[hi])
// laid out so that every lane sees x of its own half and of the other half.
__device__ __forceinline__ float halves_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Round-robin dispatch puts workgroup b on XCD b % 8. Remap so that each XCD
// walks one contiguous range of the logical work order (shared K/V stays in
// that XCD's L2). A bijection on [0, n).
__device__ __forceinline__ int xcd_remap(int b, int n) {
    const int per = n >> 3;
    const int full = per << 3;
    if (b >= full) return b;
    return (b & 7) * per + (b >> 3);
}

}  // namespace hta
