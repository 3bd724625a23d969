// win_attn.hip -- frame-windowed block-causal softmax attention (SWA and DSWA).
//
// Method: page "Kairos：面向物理 AI 的原生世界模型栈" (yingwang.github.io), section
// 二、方法, second pillar: SWA is standard attention inside a window of W frames
// (L x window_size tokens, L tokens per frame); DSWA keeps the window size but
// spaces its taps `dilation` frames apart (the page realises it by regrouping
// (B, F*L, D) -> (B*d, F/d*L, D); here the regrouping is an index map over
// tap frames and is never materialised). A query attends to every key of each
// tap frame, its own frame included, and to no later frame.
//
// bf16 kernel (d = 128), one workgroup = 4 waves = 128 query rows of one frame:
//   * each wave keeps its 32 query rows as MFMA B fragments in registers and
//     computes S^T = K Q^T (keys x queries) with v_mfma_f32_32x32x16_bf16, so a
//     lane owns one query and 16 of its logits per 32-key block: the softmax
//     row max / sum is lane-local plus one swap with lane^32;
//   * O^T += V^T P^T reuses the logits' register layout directly as the B
//     fragment (key order permuted consistently in both operands), so P never
//     goes through LDS;
//   * key/value tiles of 64 keys stream into a two-stage LDS ring with direct
//     global->LDS loads (16 bytes per lane, no register round trip), issued
//     one tile ahead; A fragments of V^T are transposed LDS reads
//     (ds_read_b64_tr_b16) of the row-major V tile;
//   * three forms (NBR): one branch per launch (the SWA pass writes its fp32
//     partial, the DSWA pass adds onto it); both branches in one launch with
//     one accumulator set (the hybrid's pass: the query's own frame, common to
//     both, is attended once, its softmax state parked in a workspace while the
//     SWA taps finish and resumed for the DSWA taps); both branches with two
//     live accumulator sets (no workspace, one wave per SIMD);
//   * running max is updated lazily (only when a logit exceeds it by more than
//     8 in log2 units), so the O rescale is rare; exp2 with the log2(e) scale
//     folded into one FMA;
//   * the softmax denominator sums the same bf16-rounded weights that feed the
//     PV product (v_dot2_f32_bf16 against ones), so the output is an exact
//     convex combination of those weights;
//   * the epilogue adds up to two fp32 partials (the other branches) and writes
//     the fp32 sum, or rounds it once to bf16.
// fp32 kernel (d = 64 or 128): a plain per-row online softmax on the vector
// ALU (4 lanes per query row); used for fp32 inputs, whose workloads are tiny.
#include <type_traits>

#include "device_common.h"
#include "hta_internal.h"
#include "win_tiles.h"

namespace hta {

namespace {

using namespace tiles;

constexpr int kBQ = 128;         // query rows per workgroup
constexpr float kLazyLog2 = 8.0f;

struct Acc {
    f32x16 o[4];   // O^T fragments: d-block db, element i -> d = 32 db + 8(i/4) + 4 h + i%4
    float m;       // running max (raw logit units)
    float l;       // this lane's share of the softmax denominator
};

__device__ __forceinline__ void acc_init(Acc& a) {
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) a.o[db][i] = 0.f;
    a.m = -INFINITY;
    a.l = 0.f;
}

// Storage index of the key frame of segment sg (branch A's present taps first).
__device__ __forceinline__ long long seg_frame(const WinLaunch& w, long long fa, int sg, int nAv) {
    const int off = sg < nAv ? w.taps.offA[sg] : w.taps.offB[sg - nAv];
    const long long f = fa - off;
    return w.R > 0 ? (f % w.R) : f;
}

// One 64-key tile for one wave: S^T = K Q^T, lazy online softmax, O^T += V^T P^T.
// Ks / Vs are the tile's LDS stage (compile-time addresses once inlined, so the
// per-lane offsets plus immediates address every fragment). A ragged tile (the
// last of a frame, nvalid < 64 keys) runs the same code with its missing keys'
// logits set to -inf: one code path touches the accumulators, so they keep
// their registers across iterations.
__device__ __forceinline__ void attend_tile(Acc& a, const bf16x8 (&qf)[8], const char* Ks,
                                            const char* Vs, const LaneOffs& L, int nvalid,
                                            float c, int lane) {
    const int h = lane >> 5;
    f32x16 s[2];
    const f32x16 zero = {};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const bf16x8 kf = *reinterpret_cast<const bf16x8*>(Ks + kb * 32 * kRowB + L.k[ks]);
            s[kb] = mfma32(kf, qf[ks], ks == 0 ? zero : s[kb]);
        }
    if (__builtin_expect(nvalid < kBK, 0)) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int key = kb * 32 + 8 * (i >> 2) + 4 * h + (i & 3);
                if (key >= nvalid) s[kb][i] = -INFINITY;
            }
    }
    float mt = s[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mt = fmaxf(mt, s[kb][i]);
    mt = halves_max(mt);
    const bool grow = (mt - a.m) * c > kLazyLog2;
    if (__any(grow)) {
        const float mn = grow ? mt : a.m;
        const float corr = fast_exp2((a.m - mn) * c);
        a.m = mn;
        a.l *= corr;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) a.o[db][i] *= corr;
    }
    const float mc = a.m * c;
    bf16x8 pf[2][2];
    float lsum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int gg = 0; gg < 2; ++gg) {
#pragma unroll
            for (int j = 0; j < 8; ++j)
                pf[kb][gg][j] = f2bf(fast_exp2(__builtin_fmaf(s[kb][8 * gg + j], c, -mc)));
            // the denominator sums the same rounded weights the PV product uses
#pragma unroll
            for (int j = 0; j < 8; j += 2)
                lsum = add_pair(bf16x2{pf[kb][gg][j], pf[kb][gg][j + 1]}, lsum);
        }
    a.l += lsum;
    typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int gg = 0; gg < 2; ++gg)
#pragma unroll
            for (int db = 0; db < 4; ++db) {
                const char* vb = Vs + (kb * 32 + 16 * gg) * kRowB;
                const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vb + L.v[db]));
                const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vb + L.vh[db]));
                a.o[db] = mfma32(cat(lo, hi), pf[kb][gg], a.o[db]);
            }
}

// Walks the tiles of a workgroup in order: segment (tap frame) sg, tile tk.
struct TileCursor {
    int sg, tk;
    const bf16* kf;   // K / V of the current segment's frame
    const bf16* vf;
};

// Parked softmax state of one wave (nbr 3): per lane 64 accumulator values, m
// and l, contiguous (68 floats, 16-byte aligned), so one address per lane plus
// immediate offsets reaches all of it.
constexpr int kParkPerLane = 68;

__device__ __forceinline__ void park_store(const Acc& a, float* p) {
    f32x4* q = reinterpret_cast<f32x4*>(p);
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g)
            q[4 * db + g] = f32x4{a.o[db][4 * g], a.o[db][4 * g + 1], a.o[db][4 * g + 2],
                                  a.o[db][4 * g + 3]};
    q[16] = f32x4{a.m, a.l, 0.f, 0.f};
}

__device__ __forceinline__ void park_load(Acc& a, const float* p) {
    const f32x4* q = reinterpret_cast<const f32x4*>(p);
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const f32x4 x = q[4 * db + g];
#pragma unroll
            for (int i = 0; i < 4; ++i) a.o[db][4 * g + i] = x[i];
        }
    const f32x4 ml = q[16];
    a.m = ml[0];
    a.l = ml[1];
}

// Two waves per SIMD for the single-accumulator kernels (NBR 1, and NBR 3 which
// parks the shared own-frame state in memory instead of keeping a second set);
// the two-set kernel (NBR 2) runs at one.
template <int NBR>
__global__ __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(NBR == 2 ? 1 : 2, NBR == 2 ? 1 : 2)))
void win_attn_bf16_kernel(WinLaunch w) {
    __shared__ __attribute__((aligned(1024))) char Kst[2][kTileB];
    __shared__ __attribute__((aligned(1024))) char Vst[2][kTileB];
    typedef __attribute__((address_space(3))) char lds_char;
    const uint32_t ldsK = (uint32_t)(uintptr_t)(lds_char*)&Kst[0][0];
    const uint32_t ldsV = (uint32_t)(uintptr_t)(lds_char*)&Vst[0][0];

    const int nqt = (w.P + kBQ - 1) / kBQ;
    const int nwg = w.BH * w.Tq * nqt;
    const int wid = xcd_remap(blockIdx.x, nwg);
    const int qt = wid % nqt;
    const int fq = w.Tq - 1 - (wid / nqt) % w.Tq;   // heavy (late) frames first
    const int bh = wid / (nqt * w.Tq);
    const long long fa = w.frame0 + fq;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = lane & 31, h = lane >> 5;
    LaneOffs L;
    lane_offsets(L, wave, lane);

    const bf16* kbh = static_cast<const bf16*>(w.k) + (long long)bh * w.kv_bh;
    const bf16* vbh = static_cast<const bf16*>(w.v) + (long long)bh * w.kv_bh;

    // Segments: present taps of branch A, then of branch B.
    const int nSegA = taps_present(w.taps.offA, w.taps.nA, fa);
    const int nseg = nSegA + (NBR >= 2 ? taps_present(w.taps.offB, w.taps.nB, fa) : 0);
    const int ntk = (w.P + kBK - 1) / kBK;
    const int nit = nseg * ntk;
    float* park = NBR == 3 ? w.park + (((size_t)wid * 4 + wave) * 64 + lane) * kParkPerLane : nullptr;

    auto seg_base = [&](TileCursor& t) {
        const long long ofs = seg_frame(w, fa, t.sg, nSegA) * w.kv_frame;
        t.kf = kbh + ofs;
        t.vf = vbh + ofs;
    };
    auto advance = [&](TileCursor& t) {
        if (++t.tk == ntk) {
            t.tk = 0;
            if (++t.sg < nseg) seg_base(t);
        }
    };
    auto issue = [&](const TileCursor& t, uint32_t stage) {
        const long long ofs = (long long)t.tk * kBK * kD;
        issue_tile(ldsK + stage * kTileB, ldsV + stage * kTileB, t.kf + ofs, t.vf + ofs,
                   min(kBK, w.P - t.tk * kBK), wave, lane, L);
    };

    TileCursor ti{0, 0, kbh, vbh};   // next tile to stage
    if (nit > 0) {
        seg_base(ti);
        issue(ti, 0);
        advance(ti);
    }

    // Query fragments (B operand of S^T = K Q^T).
    const int qrow = qt * kBQ + wave * 32 + n;
    const bool wave_rows = qt * kBQ + wave * 32 < w.P;
    const bf16* qp = static_cast<const bf16*>(w.q) + (long long)bh * w.q_bh + ((long long)fq * w.P + qrow) * kD;
    bf16x8 qf[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
        if (qrow < w.P) qf[ks] = *reinterpret_cast<const bf16x8*>(qp + 16 * ks + 8 * h);
        else
#pragma unroll
            for (int j = 0; j < 8; ++j) qf[ks][j] = (bf16)0.f;
    }
    const float c = w.scale * kLog2e;

    Acc A, Bacc;
    acc_init(A);
    acc_init(Bacc);

    int sg = 0, tk = 0;   // tile being consumed
    // One tile in stage ST (compile-time, so LDS addresses fold into immediates).
    auto step = [&](int it, auto stage_tag) __attribute__((always_inline)) {
        constexpr int ST = decltype(stage_tag)::value;
        wait_vmcnt<0>();   // this tile's loads (issued one tile ago) have landed ...
        __syncthreads();   // ... for every wave; and the stage refilled next was read by all
        if (it + 1 < nit) {
            issue(ti, ST ^ 1);
            advance(ti);
        }
        const int nvalid = min(kBK, w.P - tk * kBK);
        if (wave_rows) {   // waves whose 32 query rows all lie past the frame only stage tiles
            Acc& acc = (NBR != 2 || sg < nSegA) ? A : Bacc;
            attend_tile(acc, qf, Kst[ST], Vst[ST], L, nvalid, c, lane);
            // own frame done: park the state branch B resumes from
            if (NBR == 3 && sg == 0 && tk == ntk - 1) park_store(A, park);
        }
        if (NBR == 2 && sg == 0 && tk == ntk - 1) Bacc = A;   // own frame seeds branch B
        if (++tk == ntk) { tk = 0; ++sg; }
    };
    // Tiles [it0, it1) with tile it in stage it & 1 (S0 = it0 & 1).
    auto run = [&](int it0, int it1, auto first_stage) __attribute__((always_inline)) {
        constexpr int S0 = decltype(first_stage)::value;
        for (int it = it0; it < it1; it += 2) {
            step(it, std::integral_constant<int, S0>{});
            if (it + 1 < it1) step(it + 1, std::integral_constant<int, S0 ^ 1>{});
        }
    };
    if (NBR == 3) {
        // Branch A's tiles (own frame first), then branch B's in a loop of their
        // own: the switch between them -- branch A's output written, the parked
        // own-frame state reloaded -- stays off the per-tile path, so the
        // accumulators keep their registers through both loops.
        const int nitA = nSegA * ntk;
        run(0, nitA, std::integral_constant<int, 0>{});
        if (wave_rows) {
            const float lA = halves_sum(A.l);
            const float inv = 1.f / lA;
            if (w.lse && h == 0 && qrow < w.P)
                w.lse[(long long)bh * w.Tq * w.P + (long long)fq * w.P + qrow] = A.m * w.scale + logf(lA);
            float* oa = w.oa + (long long)bh * w.q_bh + ((long long)fq * w.P + qrow) * kD;
            if (qrow < w.P) {
#pragma unroll
                for (int db = 0; db < 4; ++db)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const int d0 = db * 32 + 8 * g + 4 * h;
                        *reinterpret_cast<f32x4*>(oa + d0) =
                            f32x4{A.o[db][4 * g] * inv, A.o[db][4 * g + 1] * inv,
                                  A.o[db][4 * g + 2] * inv, A.o[db][4 * g + 3] * inv};
                    }
            }
            park_load(A, park);
        }
        if (nitA & 1) run(nitA, nit, std::integral_constant<int, 1>{});
        else run(nitA, nit, std::integral_constant<int, 0>{});
    } else {
        run(0, nit, std::integral_constant<int, 0>{});
    }

    // Epilogue: o = O_A / l_A (+ O_B / l_B) (+ add) (+ add2), rounded once.
    if (qrow >= w.P) return;
    const float lA = halves_sum(A.l);
    const float invA = 1.f / lA;
    // log-sum-exp of the scaled logits: the weights summed in l are
    // exp(scale (s - m)), m in raw logit units
    if (NBR == 1 && w.lse && h == 0)
        w.lse[(long long)bh * w.Tq * w.P + (long long)fq * w.P + qrow] = A.m * w.scale + logf(lA);
    if (NBR == 3 && w.lse2 && h == 0)   // branch B's (the resumed state's)
        w.lse2[(long long)bh * w.Tq * w.P + (long long)fq * w.P + qrow] = A.m * w.scale + logf(lA);
    float invB = 0.f;
    if (NBR == 2) invB = 1.f / halves_sum(Bacc.l);
    const long long orow = (long long)bh * w.q_bh + ((long long)fq * w.P + qrow) * kD;
    const float* ap = w.add ? w.add + orow : nullptr;
    const float* ap2 = w.add2 ? w.add2 + orow : nullptr;
    const float* apa = NBR == 3 ? w.oa + orow : nullptr;   // branch A's output
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int d0 = db * 32 + 8 * g + 4 * h;
            float r[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                r[i] = A.o[db][4 * g + i] * invA;
                if (NBR == 2) r[i] += Bacc.o[db][4 * g + i] * invB;
            }
            if ((NBR == 1 || NBR == 3) && w.obr)   // this branch's (nbr 3: branch B's) output
                *reinterpret_cast<f32x4*>(w.obr + orow + d0) = f32x4{r[0], r[1], r[2], r[3]};
            if (NBR == 3) {
                const f32x4 x = *reinterpret_cast<const f32x4*>(apa + d0);
#pragma unroll
                for (int i = 0; i < 4; ++i) r[i] += x[i];
            }
            if (ap) {
                const f32x4 x = *reinterpret_cast<const f32x4*>(ap + d0);
#pragma unroll
                for (int i = 0; i < 4; ++i) r[i] += x[i];
            }
            if (ap2) {
                const f32x4 x = *reinterpret_cast<const f32x4*>(ap2 + d0);
#pragma unroll
                for (int i = 0; i < 4; ++i) r[i] += x[i];
            }
            if (w.out_f32) {
                *reinterpret_cast<f32x4*>(static_cast<float*>(w.o) + orow + d0) =
                    f32x4{r[0], r[1], r[2], r[3]};
            } else {
                bf16x4 ov;
#pragma unroll
                for (int i = 0; i < 4; ++i) ov[i] = f2bf(r[i]);
                *reinterpret_cast<bf16x4*>(static_cast<bf16*>(w.o) + orow + d0) = ov;
            }
        }
}

// ---------------------------------------------------------------------------------
// fp32 path: 64 query rows per workgroup, 4 lanes per row (each owns D/4 dims,
// interleaved), keys streamed from global memory, exact online softmax.

template <int D>
__device__ __forceinline__ void f32_branch(const WinLaunch& w, long long fa, int nAv,
                                           const float* qv, const float* kbh, const float* vbh,
                                           int s0, int s1, int sub,
                                           float& m, float& l, float (&acc)[D / 4]) {
    const int P = w.P;
    const float scale = w.scale;
    for (int sg = s0; sg < s1; ++sg) {
        const long long fr = seg_frame(w, fa, sg, nAv);
        const float* kf = kbh + fr * w.kv_frame;
        const float* vf = vbh + fr * w.kv_frame;
        for (int p = 0; p < P; ++p) {
            const float* kr = kf + (long long)p * D;
            float s = 0.f;
#pragma unroll
            for (int i = 0; i < D / 4; ++i) s += qv[i] * kr[4 * i + sub];
            s += __shfl_xor(s, 1, 64);
            s += __shfl_xor(s, 2, 64);
            s *= scale;
            const float mn = fmaxf(m, s);
            const float corr = expf(m - mn);
            const float e = expf(s - mn);
            l = l * corr + e;
            const float* vr = vf + (long long)p * D;
#pragma unroll
            for (int i = 0; i < D / 4; ++i) acc[i] = acc[i] * corr + e * vr[4 * i + sub];
            m = mn;
        }
    }
}

template <int D, int NBR>
__global__ __launch_bounds__(256) void win_attn_f32_kernel(WinLaunch w) {
    const int nqt = (w.P + 63) / 64;
    const int wid = blockIdx.x;
    const int qt = wid % nqt;
    const int fq = (wid / nqt) % w.Tq;
    const int bh = wid / (nqt * w.Tq);
    const long long fa = w.frame0 + fq;
    const int sub = threadIdx.x & 3;
    const int row = qt * 64 + (threadIdx.x >> 2);
    const bool valid = row < w.P;
    const int prow = valid ? row : w.P - 1;   // invalid rows compute a duplicate, never stored

    const int nSegA = taps_present(w.taps.offA, w.taps.nA, fa);
    const int nseg = nSegA + (NBR == 2 ? taps_present(w.taps.offB, w.taps.nB, fa) : 0);

    const float* kbh = static_cast<const float*>(w.k) + (long long)bh * w.kv_bh;
    const float* vbh = static_cast<const float*>(w.v) + (long long)bh * w.kv_bh;
    const long long qoff = (long long)bh * w.q_bh + ((long long)fq * w.P + prow) * D;
    const float* qp = static_cast<const float*>(w.q) + qoff;
    float qv[D / 4];
#pragma unroll
    for (int i = 0; i < D / 4; ++i) qv[i] = qp[4 * i + sub];

    float accA[D / 4], accB[D / 4];
#pragma unroll
    for (int i = 0; i < D / 4; ++i) { accA[i] = 0.f; accB[i] = 0.f; }
    float mA = -INFINITY, lA = 0.f, mB = -INFINITY, lB = 0.f;
    if (NBR == 2) {
        // Own frame once, then both branches continue from that state.
        f32_branch<D>(w, fa, nSegA, qv, kbh, vbh, 0, 1, sub, mA, lA, accA);
        mB = mA; lB = lA;
#pragma unroll
        for (int i = 0; i < D / 4; ++i) accB[i] = accA[i];
        f32_branch<D>(w, fa, nSegA, qv, kbh, vbh, 1, nSegA, sub, mA, lA, accA);
        f32_branch<D>(w, fa, nSegA, qv, kbh, vbh, nSegA, nseg, sub, mB, lB, accB);
    } else {
        f32_branch<D>(w, fa, nSegA, qv, kbh, vbh, 0, nseg, sub, mA, lA, accA);
    }
    if (!valid) return;
    if (NBR == 1 && w.lse && sub == 0)
        w.lse[(long long)bh * w.Tq * w.P + (long long)fq * w.P + row] = mA + logf(lA);
    float* op = static_cast<float*>(w.o) + qoff;
    const float* ap = w.add ? w.add + qoff : nullptr;
    const float* ap2 = w.add2 ? w.add2 + qoff : nullptr;
    const float iA = 1.f / lA;
    const float iB = NBR == 2 ? 1.f / lB : 0.f;
#pragma unroll
    for (int i = 0; i < D / 4; ++i) {
        float r = accA[i] * iA;
        if (NBR == 2) r += accB[i] * iB;
        if (NBR == 1 && w.obr) w.obr[qoff + 4 * i + sub] = r;
        if (ap) r += ap[4 * i + sub];
        if (ap2) r += ap2[4 * i + sub];
        op[4 * i + sub] = r;
    }
}

}  // namespace

size_t win_attn_park_bytes(int BH, int Tq, int P) {
    const long long nwg = (long long)BH * Tq * ((P + kBQ - 1) / kBQ);
    return (size_t)nwg * 4 * kParkPerLane * 64 * sizeof(float);
}

hipError_t launch_win_attn(const WinLaunch& w, hipStream_t stream) {
    if (w.BH == 0 || w.Tq == 0 || w.P == 0) return hipSuccess;
    if (w.dtype == 1) {  // bf16, d == 128
        const int nqt = (w.P + kBQ - 1) / kBQ;
        const long long nwg = (long long)w.BH * w.Tq * nqt;
        if (nwg > 0x7fffffffLL) return hipErrorInvalidValue;
        if (w.nbr == 3) {
            if (!w.park || !w.oa) return hipErrorInvalidValue;
            hipLaunchKernelGGL((win_attn_bf16_kernel<3>), dim3((unsigned)nwg), dim3(256), 0, stream, w);
        } else if (w.nbr == 2)
            hipLaunchKernelGGL((win_attn_bf16_kernel<2>), dim3((unsigned)nwg), dim3(256), 0, stream, w);
        else
            hipLaunchKernelGGL((win_attn_bf16_kernel<1>), dim3((unsigned)nwg), dim3(256), 0, stream, w);
        return hipGetLastError();
    }
    const int nqt = (w.P + 63) / 64;
    const long long nwg = (long long)w.BH * w.Tq * nqt;
    if (nwg > 0x7fffffffLL) return hipErrorInvalidValue;
    const dim3 g((unsigned)nwg), b(256);
    if (w.d == 64) {
        if (w.nbr == 2) hipLaunchKernelGGL((win_attn_f32_kernel<64, 2>), g, b, 0, stream, w);
        else hipLaunchKernelGGL((win_attn_f32_kernel<64, 1>), g, b, 0, stream, w);
    } else {
        if (w.nbr == 2) hipLaunchKernelGGL((win_attn_f32_kernel<128, 2>), g, b, 0, stream, w);
        else hipLaunchKernelGGL((win_attn_f32_kernel<128, 1>), g, b, 0, stream, w);
    }
    return hipGetLastError();
}

}  // namespace hta
