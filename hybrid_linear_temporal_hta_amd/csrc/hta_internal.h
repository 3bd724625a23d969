// hta_internal.h -- launcher interface between the C-ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace hta {

constexpr int kMaxTaps = 16;

// Frame offsets of one windowed-attention launch. Branch A's offsets are
// processed first; with two branches, offset 0 (the query's own frame) is
// listed once, first in A, and its partial softmax state seeds branch B too.
struct WinTaps {
    int nA, nB;
    int offA[kMaxTaps];
    int offB[kMaxTaps];
};

// One windowed-attention launch (SWA, DSWA, or both summed).
//   query frame fq (0..Tq-1) has absolute frame index frame0 + fq;
//   key frame for offset j is abs - j, skipped if < 0;
//   key frame storage index is abs - j (linear) or (abs - j) mod R (ring).
struct WinLaunch {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    const float* add;       // optional fp32 partial [BH][Tq*P][dv] added to o (may equal o for fp32)
    const float* add2;      // optional second fp32 partial, same layout (never equals o)
    long long q_bh;         // elements between (b,h) slices of q / o / add
    long long kv_bh;        // elements between (b,h) slices of k / v
    long long kv_frame;     // elements between consecutive key frames (P*d)
    int BH, P, Tq;
    long long frame0;
    int R;                  // 0 = linear key addressing
    float scale;            // softmax scale
    int d;                  // dk == dv
    int dtype;              // HTA_F32 / HTA_BF16 (inputs)
    int out_f32;            // 1: o is fp32, 0: o is bf16
    int nbr;                // 1 or 2 branches, or 3: both branches with one accumulator
                            //   set (bf16): the own frame's state is parked in `park`
                            //   and resumed for branch B after branch A is written to `oa`
    WinTaps taps;
    float* lse;             // optional [BH][Tq*P]: log-sum-exp of the scaled logits (one
                            //   branch; nbr 3: branch A's)
    float* lse2;            // nbr 3, optional: branch B's log-sum-exp
    float* obr;             // optional fp32 [BH][Tq*P][dv]: this branch's own output (one
                            //   branch; nbr 3: branch B's)
    float* park;            // nbr 3: scratch, win_attn_park_bytes(BH, Tq, P) bytes
    float* oa;              // nbr 3: fp32 [BH][Tq*P][dv] for branch A's output (may be o when
                            //   o is fp32 and no partial is added in place)
};
size_t win_attn_park_bytes(int BH, int Tq, int P);

// dst = a + b elementwise (fp32), written as fp32 or rounded to bf16; n a multiple of 4.
hipError_t launch_add_f32(void* dst, int dst_bf16, const float* a, const float* b, long long n,
                          hipStream_t stream);

hipError_t launch_win_attn(const WinLaunch& w, hipStream_t stream);

// Backward of one windowed-attention branch over a whole sequence (no ring).
// Per-row statistics {lse * log2(e), D = dO . o} come first (launch_win_bwd_prep),
// then the query pass (dq) and the key pass (dk, dv).
struct BwdPrep {
    const void* o;          // branch output [rows][d], fp32 or bf16
    const void* dout;       // dL/do [rows][d], fp32 or bf16
    const float* lse;       // [rows]
    float* stats;           // out: [rows][2] = {lse * log2(e), D}
    void* dout_bf16;        // optional out: dout rounded to bf16 (fp32 dout, bf16 inputs)
    long long rows;
    int d;
    int o_f32, do_f32;
    int round_do;           // D from the bf16-rounded dout (what the bf16 kernels multiply)
    // bf16 inputs only (optional):
    const void* q;          // q, k [rows][d] bf16: copied to fp16 into q16, k16
    const void* k;
    void* q16;
    void* k16;
    const void* v;          // v [rows][d] bf16: max |v| into gmax[1]
    unsigned* gmax;         // float bits, zeroed before: max |dout| (as rounded), max |v|,
                            //   and (with q16) max |q|, max |k| -- the copies' scales
};
hipError_t launch_win_bwd_prep(const BwdPrep& p, hipStream_t stream);

struct BwdLaunch {
    const void* q;
    const void* k;
    const void* v;
    const void* dout;       // dtype of q (bf16 dout for bf16 inputs)
    const float* stats;     // [BH][L][2] from the prep, 64 rows of padding after the end
    void* dq;
    void* dk;
    void* dv;
    const float* add_q;     // optional fp32 partials [BH][L][d] added before the store
    const float* add_k;
    const float* add_v;
    const float* add2_q;    // optional second set of partials (never equal to the outputs)
    const float* add2_k;
    const float* add2_v;
    int out_f32;            // gradients written as fp32 (1) or bf16 (0)
    long long bh_elems;     // elements between (b,h) slices (L*d)
    int BH, P, T, d, dtype;
    float scale;
    int ntaps;
    int off[kMaxTaps];      // ascending frame offsets: query frame f reads key frames f - off[j]
    // bf16 path: fp16 copies 2^eq q and 2^ek k and the maxima that fix those
    // powers of two and the one of dS in its fp16 products (gmax[0..3])
    const void* q16;
    const void* k16;
    const unsigned* gmax;
};
constexpr int kBwdQuery = 1, kBwdKey = 2;
hipError_t launch_win_bwd(const BwdLaunch& b, hipStream_t stream, int parts = kBwdQuery | kBwdKey);

// Chunked GLA over one segment of tokens per (b,h).
struct GlaLaunch {
    const void* q;
    const void* k;
    const void* v;
    const float* alpha;
    const float* beta;
    float* state;           // [BH][d][d] in/out
    void* o;                // output; may be NULL (state only)
    int out_f32;            // 1: o is fp32, 0: o is bf16
    long long L;            // tokens per (b,h)
    int BH, d, chunk;
    float scale;
    int dtype;
    int form;               // 0: GatedDeltaNet reading, 1: the printed update (erase not gated)
    void* ring_k;           // optional (bf16 prep): k and v of these tokens are also copied,
    void* ring_v;           //   unchanged, to ring + bh * ring_bh + ring_off + token * d
    long long ring_bh;      // elements between (b,h) slices of the ring
    long long ring_off;     // element offset of the slot inside a (b,h) slice
    void* ws;               // workspace
    size_t ws_bytes;
    void* save_m;           // optional fp16 [BH][nch][d][d]: the state entering each chunk
    void* save_u;           // optional fp16 [BH][nch][64][d]: each chunk's U (bf16 path)
    const unsigned* vscale; // optional (saving scan): float bits of max(|v|, |state|); the scan
                            //   runs on v and the state times the power of two that maps it
                            //   into [1, 2) (saved M0, U carry the factor; o and the final
                            //   state do not)
};

// Backward of the GLA branch over one sequence per (b,h): given dL/do and
// dL/dM_L (in dstate), the gradients of q, k, v, alpha, beta and dL/dM_0 (out
// in dstate). The forward is recomputed from the inputs and the initial state.
struct GlaBwdLaunch {
    const void* q;
    const void* k;
    const void* v;
    const float* alpha;
    const float* beta;
    const float* state0;    // [BH][d][d] initial state M_0 = S_0^T
    const void* dout;       // [BH][L][d], fp32 (do_f32) or bf16
    int do_f32;
    float* dstate;          // [BH][d][d]: in dL/dM_L, out dL/dM_0
    void* dq;               // dtype of q
    void* dk;
    void* dv;
    float* dalpha;          // [BH][L]
    float* dbeta;
    long long L;
    int BH, d, chunk;
    float scale;            // output scale of the forward
    int dtype;
    int form;               // 0: GatedDeltaNet reading, 1: the printed update
    int grad_f32;           // bf16 inputs: write dq, dk, dv as fp32 (partials of a sum)
    void* ws;
    size_t ws_bytes;
};
size_t gla_bwd_workspace_bytes(int dtype, int BH, long long L, int d);
hipError_t launch_gla_bwd(const GlaBwdLaunch& b, hipStream_t stream);

// Per-token projections and gates (bf16 MFMA GEMM + fused epilogue).
struct ProjLaunch {
    const void* x;          // [M][Dm] bf16, M = B * L tokens
    const void* w;          // [Dm][N] bf16, N = 3 * H * 128 + 2 * H
    void* q;                // [B][H][L][128] bf16
    void* k;
    void* v;
    float* alpha;           // [B][H][L] fp32
    float* beta;
    long long M, L;
    int Dm, N, H;
    int flags;              // bit 0: L2-normalise q, bit 1: L2-normalise k
    long long nmt;          // token tiles of 128
};
hipError_t launch_project(const ProjLaunch& p, hipStream_t stream);

// Chunked GLA: fp32 (vector ALU) and bf16 (MFMA) paths.
hipError_t launch_gla_f32(const GlaLaunch& g, hipStream_t stream);
// bf16 GLA: the chunk-parallel prep kernel, then the sequential scan kernel
// (parts selects either or both, so the two can go on different streams).
constexpr int kGlaPrep = 1, kGlaScan = 2;
hipError_t launch_gla_bf16(const GlaLaunch& g, hipStream_t stream, int parts = kGlaPrep | kGlaScan);
size_t gla_bf16_workspace_bytes(int BH, long long L, int chunk);
// The bf16 forward (prep with per-chunk power-of-two operand scales, then the
// chunk scan); o may be NULL (state only). parts: kGlaPrep and / or one scan
// shape, kGlaScan (the whole chip) or kGlaScanNarrow (few compute units, to run
// beside other work).
constexpr int kGlaScanNarrow = 4;
hipError_t launch_gla_fwd(const GlaLaunch& g, hipStream_t stream, int parts = kGlaPrep | kGlaScan);
size_t gla_fwd_workspace_bytes(int BH, long long L);
// Chunk operand block of the bf16 path (bytes per 64-token chunk).
size_t gla_bf16_chunk_bytes();

// Per-(b,h) strided copy of `elems` elements (16-byte multiples) from
// src[bh*src_bh + src_off] to dst[bh*dst_bh + dst_off] (strides/offsets in elements).
hipError_t launch_copy_frames(const void* src, void* dst, int BH, long long src_bh,
                              long long dst_bh, long long src_off, long long dst_off,
                              long long elems, int elem_bytes, hipStream_t stream);

// dst[i] = src ? src[i] : 0 for i < n (a kernel, not hipMemsetAsync).
hipError_t launch_fill_f32(float* dst, const float* src, long long n, hipStream_t stream);

}  // namespace hta
