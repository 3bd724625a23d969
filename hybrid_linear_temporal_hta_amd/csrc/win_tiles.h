// win_tiles.h -- pieces shared by the bf16 windowed-attention kernels (forward
// and backward): tile geometry, the LDS swizzle, direct global->LDS staging of
// 64-row tiles and the per-lane fragment offsets into a staged tile.
//
// A staged tile holds 64 rows of 128 bf16 (256 bytes per row, unpadded). Its
// 16-byte chunk c of row r lives in slot c ^ swz(r). Two reads address it:
//   * row fragments (MFMA A or B operand with the contraction along the row):
//     lane l reads 16 bytes of row l % 32 -- LaneOffs::k;
//   * transposed fragments (contraction along the rows): ds_read_b64_tr_b16
//     of 4 rows x 4 columns per 16 lanes -- LaneOffs::v / vh.
#pragma once

#include "device_common.h"
#include "hta_internal.h"
#include "lds_dma.h"

namespace hta {
namespace tiles {

constexpr int kD = 128;          // head dim of the bf16 kernels
constexpr int kBK = 64;          // rows per staged LDS tile
constexpr int kRowB = kD * 2;    // bytes per staged row (unpadded, chunk-swizzled)
constexpr int kTileB = kBK * kRowB;

// 16-byte chunk c of LDS row r lives in slot c ^ swz(r), a rotation of the row's
// low four bits: on gfx950's 64-bank LDS this is conflict-free for both the K
// fragment reads (32 rows x one chunk) and the transposed V reads (4 rows x 4
// chunks per 16 lanes), as the SQ_LDS_BANK_CONFLICT counter confirms.
__device__ __forceinline__ int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

// Offsets are ascending, so the taps present for absolute query frame fa
// (those with fa - off >= 0) are a prefix of each list.
__device__ __forceinline__ int taps_present(const int* off, int n, long long fa) {
    int c = 0;
    for (int j = 0; j < n; ++j) c += (off[j] <= fa) ? 1 : 0;
    return c;
}

// Transposed LDS reads (ds_read_b64_tr_b16) of 16-bit elements, as bf16 or fp16.
__device__ __forceinline__ bf16x4 tr_bf16(const char* p) {
    typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)p);
}
__device__ __forceinline__ f16x4 tr_f16(const char* p) {
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    return __builtin_bit_cast(f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p));
}

// Per-lane byte offsets that stay fixed for the whole kernel.
struct LaneOffs {
    uint32_t k[8];     // row fragment ks of row n (32-row block 0, stage 0)
    uint32_t v[4];     // transposed fragment of d-block db, rows 4(g/2) + j (block 0, stage 0)
    uint32_t vh[4];    // ... and rows 8 + 4(g/2) + j (swz differs in row bit 3)
};

// Row and column of the chunk that DMA instruction i of `wave` fills for `lane`:
// chunk 64 (4 wave + i) + lane = row r, slot c ^ swz(r).
__device__ __forceinline__ int dma_row(int wave, int i, int lane) { return (64 * (4 * wave + i) + lane) >> 4; }
__device__ __forceinline__ int dma_col(int wave, int i, int lane) {
    const int p = 64 * (4 * wave + i) + lane;
    return ((p & 15) ^ swz(p >> 4)) * 8;
}

__device__ __forceinline__ void lane_offsets(LaneOffs& L, int wave, int lane) {
    const int n = lane & 31, h = lane >> 5;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) L.k[ks] = n * kRowB + 16 * ((2 * ks + h) ^ swz(n));
    // Transposed fragments (e.g. V^T) by transposed LDS reads: within each
    // 16-lane group g, lane 4j + a addresses row 4(g/2) + j (+8, +16 gg, +32 kb: immediates),
    // columns 16(g%2) + 4a .. +3 of the d-block; the read hands lane 4a + b
    // column b of rows j = 0..3. swz depends on row bits 0-3 only, so rows
    // +16 and +32 share these offsets and rows +8 get their own.
    const int g = lane >> 4, sl = lane & 15, jr = sl >> 2, ac = sl & 3;
    const int r0 = 4 * (g >> 1) + jr, r1 = r0 + 8;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
        const int col = 32 * db + 16 * (g & 1) + 4 * ac;
        L.v[db] = r0 * kRowB + 16 * ((col >> 3) ^ swz(r0)) + 8 * ((col >> 2) & 1);
        L.vh[db] = r1 * kRowB + 16 * ((col >> 3) ^ swz(r1)) + 8 * ((col >> 2) & 1);
    }
}

// Enqueue one 64-row tile of each of two tensors straight into LDS (K and V in
// the forward and query passes, Q and dO in the key pass). Rows past the frame's
// end (ragged tile) re-read the last valid row: finite values, masked by the caller.
// `wave` is the staging wave's index 0..3 (four waves fill a tile).
__device__ __forceinline__ void issue_tile(uint32_t ldsK, uint32_t ldsV, const bf16* kb,
                                           const bf16* vb, int nvalid, int wave, int lane,
                                           const LaneOffs& L) {
    if (nvalid == kBK) {
        // wave w, instruction i fills LDS chunks [64 (4w + i), +64) of a tile (source
        // offsets recomputed here rather than held in registers)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t off = 1024u * (4 * wave + i);
            const uint32_t src = (uint32_t)(dma_row(wave, i, lane) * kD + dma_col(wave, i, lane)) * 2;
            dma16(src, kb, ldsK + off);
            dma16(src, vb, ldsV + off);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t off = 1024u * (4 * wave + i);
            const uint32_t src =
                (uint32_t)(min(dma_row(wave, i, lane), nvalid - 1) * kD + dma_col(wave, i, lane)) * 2;
            dma16(src, kb, ldsK + off);
            dma16(src, vb, ldsV + off);
        }
    }
}

}  // namespace tiles
}  // namespace hta
