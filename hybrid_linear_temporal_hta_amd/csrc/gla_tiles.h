// gla_tiles.h -- the chunk operand block of the bf16 GLA path and the MFMA
// fragment readers over it, shared by the forward (prep, scan) and backward
// (reverse scan, chunk gradients) kernels.
//
// One 64-token chunk's block: K and Q in fp16 (exact copies of the bf16 inputs),
// T = (I + A)^-1 and Pm in fp16, and per-token fp32 factors, laid out exactly as
// the scans stage it in LDS (bank-conflict-free swizzles included).
#pragma once

#include "device_common.h"
#include "hta_internal.h"
#include "lds_dma.h"

namespace hta {
namespace glat {

constexpr int kC = 64;                 // chunk
constexpr int kD = 128;                // head dim
constexpr float kLogFloor = -1.0e4f;   // log(alpha) floor: alpha = 0 decays to exactly 0

// Operand block of one chunk (workspace and LDS stage share this layout).
constexpr int kOffK = 0;               // K fp16 [64][128], 16-byte chunks swizzled by swz64
constexpr int kOffQ = 16384;           // Q fp16, same layout
constexpr int kOffT = 32768;           // T fp16 [64][64], chunks swizzled by swz32
constexpr int kOffP = 40960;           // Pm fp16, same layout
constexpr int kOffE = 49152;           // e^{g_t} fp32 [64]
constexpr int kOffD = 49408;           // e^{g_C - g_t} fp32 [64]
constexpr int kOffB = 49664;           // beta fp32 [64] (0 past the end of the sequence)
constexpr int kOffX = 49920;           // e^{gp_t} fp32 [64]: scale of K M0 in X (gp = g, or
                                       // g_{t-1} for the printed form)
constexpr int kBlockMain = 49152;      // K, Q, T, Pm: 48 KiB = 12 x 4 KiB
constexpr int kTailChunks = 64;        // eg, ed, beta, egp: 1 KiB = 64 x 16
constexpr size_t kChunkBytes = 50176;  // + eg, ed, beta, egp
constexpr int kOffV = 50176;           // LDS only: V tile bf16 [64 tokens][64 columns]
constexpr int kStageBytes = kOffV + 64 * 64 * 2;   // 58368

// 256-byte rows (K, Q): chunk c of row r in slot c ^ swz64(r).
__device__ __forceinline__ int swz64(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
// 128-byte rows (T, Pm): chunk c of row r in slot c ^ swz32(r).
__device__ __forceinline__ int swz32(int r) { return (r >> 1) & 7; }
// 128-byte rows of the V tile.
__device__ __forceinline__ int swzv(int r) { return 2 * ((r >> 2) & 3); }

__device__ __forceinline__ int offK(int row, int col) {   // byte offset of element (row, col)
    return row * 256 + 16 * ((col >> 3) ^ swz64(row)) + 2 * (col & 7);
}
__device__ __forceinline__ int offT(int row, int col) {
    return row * 128 + 16 * ((col >> 3) ^ swz32(row)) + 2 * (col & 7);
}

// A fragment of a 16-row block from a swizzled fp16 tile: row `row`, k-step
// columns 32*ks + 4G + j (j < 4) and 32*ks + 16 + 4G + (j - 4).
__device__ __forceinline__ f16x8 afragK(const char* base, int row, int ks, int G) {
    const int c0 = 32 * ks + 4 * G;
    return cat(*reinterpret_cast<const f16x4*>(base + offK(row, c0)),
               *reinterpret_cast<const f16x4*>(base + offK(row, c0 + 16)));
}
__device__ __forceinline__ f16x8 afragT(const char* base, int row, int ks, int G) {
    const int c0 = 32 * ks + 4 * G;
    return cat(*reinterpret_cast<const f16x4*>(base + offT(row, c0)),
               *reinterpret_cast<const f16x4*>(base + offT(row, c0 + 16)));
}
// K^T fragment for d-block kb, k-step kt (tokens 32kt + 4G + j, + 16) by two
// transposed reads: source lane 4j + a addresses token row 32kt + 4G + j,
// columns 16kb + 4a .. +3; lane 4a + b receives column b of rows j = 0..3.
__device__ __forceinline__ f16x8 afragKt(const char* Kbase, int kb, int kt, int lane) {
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    const int G = lane >> 4, s = lane & 15, j = s >> 2, a = s & 3;
    const int t0 = 32 * kt + 4 * G + j;
    const int col = 16 * kb + 4 * a;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(Kbase + offK(t0, col)));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(Kbase + offK(t0 + 16, col)));
    return cat(__builtin_bit_cast(f16x4, lo), __builtin_bit_cast(f16x4, hi));
}

// B fragment from two 16x16 accumulator tiles (rows 32ks..+15 and 32ks+16..+31).
__device__ __forceinline__ f16x8 bfrag(const f32x4& lo, const f32x4& hi) {
    f16x8 b;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        b[i] = (f16)lo[i];
        b[4 + i] = (f16)hi[i];
    }
    return b;
}

// Transposed A fragment of a 64x64 swizzled fp16 matrix X (T or Pm): rows
// 16 rb + m of X^T (= columns of X), k-step kt over X's rows in the order the
// other fragments use (32 kt + 4G + j, then + 16), by two transposed reads.
__device__ __forceinline__ f16x8 afragTt(const char* base, int rb, int kt, int lane) {
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    const int G = lane >> 4, s = lane & 15, j = s >> 2, a = s & 3;
    const int t0 = 32 * kt + 4 * G + j;
    const int col = 16 * rb + 4 * a;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + offT(t0, col)));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + offT(t0 + 16, col)));
    return cat(__builtin_bit_cast(f16x4, lo), __builtin_bit_cast(f16x4, hi));
}

// Lane l reads lane l ^ 1 (resp. l ^ 2) of its quad: DPP quad permutes.
__device__ __forceinline__ float quad_xor1(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float quad_xor2(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, false));
}

// 16x16x16 fp32 product on v_mfma_f32_16x16x4_f32: acc += X Y for 16x16 blocks X
// (row stride xld) and Y (row stride yld) in LDS; lane l ends with rows
// 4 (l / 16) + i of column l % 16.
__device__ __forceinline__ f32x4 mm16f(const float* X, int xld, const float* Y, int yld,
                                       f32x4 acc, int lane) {
    const int m = lane & 15, g = lane >> 4;
#pragma unroll
    for (int s = 0; s < 4; ++s)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(X[m * xld + 4 * s + g], Y[(4 * s + g) * yld + m],
                                                   acc, 0, 0, 0);
    return acc;
}

// Power of two sigma with max * sigma in [1, 2) (1 when the max is 0).
__device__ __forceinline__ float sigma_of(unsigned bits) {
    // zero, or an inf / NaN maximum (a non-finite input): no scaling, so finite
    // operands keep their values and the non-finite one propagates
    if (bits == 0u || bits >= 0x7f800000u) return 1.f;
    const int e = (int)((bits >> 23) & 0xffu) - 127;
    return ldexpf(1.f, -max(-126, min(e, 126)));
}

}  // namespace glat
}  // namespace hta
