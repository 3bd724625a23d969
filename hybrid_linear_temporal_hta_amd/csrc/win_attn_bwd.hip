// win_attn_bwd.hip -- backward pass of frame-windowed softmax attention (SWA, DSWA).
//
// The forward is the SWA / DSWA paragraphs of page "Kairos：面向物理 AI 的原生世界
// 模型栈" (yingwang.github.io), section 二、方法, second pillar: query t in frame f
// attends to every key of the frames f - off[j] (off = 0..W-1 for SWA, j*dilation
// for DSWA). Its gradient is the chain rule through softmax; with the forward's
// per-row log-sum-exp lse_t and D_t = dO_t . o_t,
//   p_ts = exp(scale q_t.k_s - lse_t),  dp_ts = dO_t . v_s,  ds_ts = p_ts (dp_ts - D_t),
//   dq_t = scale sum_s ds_ts k_s,  dk_s = scale sum_t ds_ts q_t,  dv_s = sum_t p_ts dO_t.
// Four launches, no atomics:
//   prep       per row: stats = {lse log2(e), D} (and dO rounded to bf16 when it
//              arrives in fp32 for bf16 inputs) -- HBM-bound, one pass;
//   query pass per 128 queries (a query frame's tile): walks the key tiles of its
//              window like the forward, recomputing S^T = K Q^T and dP^T = V dO^T,
//              and accumulates dQ^T += K^T dS^T -- three MFMA products per tile;
//   key pass   per 128 keys of one key frame: walks the query tiles of every frame
//              whose window holds that key frame (f_k + off[j] < T), recomputing
//              S = Q K^T and dP = dO V^T, and accumulates dV^T += dO^T P and
//              dK^T += Q^T dS (dK and dV in two launches, S computed by both).
// dS enters its products (dQ = K^T dS, dK = Q^T dS) in fp16, against fp16
// copies of K and Q made by the prep: a bf16 dS costs about 1 % of RMS in dq and
// dk, because sum_s ds_s = 0 makes those sums cancel; fp16 keeps 11 significant
// bits. Every fp16 operand carries a power of two (exact: it changes no
// rounding): the copies are 2^eq q and 2^ek k, with max |2^eq q|, |2^ek k| in
// [8, 16) (a max pass over q and k runs first), so any finite bf16 q and k fit;
// the logits formed from them are scaled back inside the exponent. dS is scaled
// by sigma from max |dO| max |v| (found by the prep) so that it sits in fp16's
// normal range whatever the gradient's magnitude; dq, dk are scaled back exactly.
// The bf16 kernels (d = 128) keep their own 32 rows (queries or keys) as MFMA B
// fragments in registers and stream the other side through a two-stage LDS
// ring with direct global->LDS loads, as the forward does; the logits' register
// layout is reused as the B operand of the next product, so P and dS never go
// through LDS. The fp32 kernels are plain vector-ALU loops for small workloads.
#include <algorithm>
#include <type_traits>

#include "device_common.h"
#include "hta_internal.h"
#include "win_tiles.h"

namespace hta {

namespace {

using namespace tiles;

constexpr int kRows = 128;   // queries (query pass) or keys (key pass) per workgroup

// ---------------------------------------------------------------------------------
// prep: stats[row] = {lse * log2(e), dO . o}; 16 lanes per row, 16 rows per
// block, the blocks strided over the grid (so that the maxima take one atomic
// pair per workgroup: same-address atomics serialise).

// Exponent e of the power of two 2^e that maps a maximum |x| (float bits) into
// [8, 16); 0 for a zero or non-finite maximum.
__device__ __forceinline__ int qk_exp(unsigned bits) {
    const float m = __uint_as_float(bits);
    if (!(m > 0.f) || !(m < __builtin_huge_valf())) return 0;
    return max(-120, min(120, 3 - (__builtin_amdgcn_frexp_expf(m) - 1)));
}

// gmax[2] = max |q|, gmax[3] = max |k| (bf16, 16 bytes per lane, one atomic pair per
// workgroup): the scales of the fp16 copies the prep makes.
__global__ __launch_bounds__(256) void win_bwd_qkmax_kernel(const bf16* q, const bf16* k, long long n8,
                                                            unsigned* gmax) {
    __shared__ float mx[2][4];
    float mq = 0.f, mk = 0.f;
    for (long long e = (long long)blockIdx.x * 256 + threadIdx.x; e < n8; e += (long long)gridDim.x * 256) {
        const bf16x8 a = reinterpret_cast<const bf16x8*>(q)[e];
        const bf16x8 b = reinterpret_cast<const bf16x8*>(k)[e];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            mq = fmaxf(mq, fabsf(bf2f(a[i])));
            mk = fmaxf(mk, fabsf(bf2f(b[i])));
        }
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        mq = fmaxf(mq, __shfl_xor(mq, m, 64));
        mk = fmaxf(mk, __shfl_xor(mk, m, 64));
    }
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) { mx[0][wave] = mq; mx[1][wave] = mk; }
    __syncthreads();
    if (threadIdx.x < 2) {
        const float* m4 = mx[threadIdx.x];
        atomicMax(gmax + 2 + threadIdx.x, __float_as_uint(fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3]))));
    }
}

template <int D>
__global__ __launch_bounds__(256) void win_bwd_prep_kernel(BwdPrep p) {
    __shared__ float mx[2][4];
    const int sub = threadIdx.x & 15, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    constexpr int E = D / 16;       // elements per lane
    const long long nblk = (p.rows + 15) / 16;
    float md = 0.f, mv = 0.f;       // running maxima of |dout| and |v|
    for (long long blk = blockIdx.x; blk < nblk; blk += gridDim.x) {
        const long long row = blk * 16 + (threadIdx.x >> 4);
        const bool ok = row < p.rows;   // whole 16-lane groups alike
        float dov[E], ov[E];
        const long long base = (ok ? row : 0) * D + sub * E;
        if (p.do_f32) {
            const float* s = static_cast<const float*>(p.dout) + base;
#pragma unroll
            for (int i = 0; i < E; ++i) dov[i] = s[i];
        } else {
            const bf16* s = static_cast<const bf16*>(p.dout) + base;
#pragma unroll
            for (int i = 0; i < E; ++i) dov[i] = bf2f(s[i]);
        }
        if (p.o_f32) {
            const float* s = static_cast<const float*>(p.o) + base;
#pragma unroll
            for (int i = 0; i < E; ++i) ov[i] = s[i];
        } else {
            const bf16* s = static_cast<const bf16*>(p.o) + base;
#pragma unroll
            for (int i = 0; i < E; ++i) ov[i] = bf2f(s[i]);
        }
        if (p.round_do) {
#pragma unroll
            for (int i = 0; i < E; ++i) dov[i] = bf2f(f2bf(dov[i]));
        }
        if (p.dout_bf16 && ok) {
            bf16* dst = static_cast<bf16*>(p.dout_bf16) + base;
#pragma unroll
            for (int i = 0; i < E; ++i) dst[i] = f2bf(dov[i]);
        }
        if (p.q16 && ok) {   // fp16 copies 2^eq q and 2^ek k (D == 128 here: 8 per lane)
            const bf16* qs = static_cast<const bf16*>(p.q) + base;
            const bf16* ks = static_cast<const bf16*>(p.k) + base;
            f16* qd = static_cast<f16*>(p.q16) + base;
            f16* kd = static_cast<f16*>(p.k16) + base;
            const float sq = ldexpf(1.f, qk_exp(p.gmax[2])), sk = ldexpf(1.f, qk_exp(p.gmax[3]));
#pragma unroll
            for (int i = 0; i < E; ++i) {
                qd[i] = (f16)(bf2f(qs[i]) * sq);
                kd[i] = (f16)(bf2f(ks[i]) * sk);
            }
        }
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < E; ++i) acc = __builtin_fmaf(dov[i], ov[i], acc);
#pragma unroll
        for (int m = 1; m < 16; m <<= 1) acc += __shfl_xor(acc, m, 64);
        if (sub == 0 && ok) {
            p.stats[2 * row] = p.lse[row] * kLog2e;
            p.stats[2 * row + 1] = acc;
        }
        if (p.gmax && ok) {
            const bf16* vs = static_cast<const bf16*>(p.v) + base;
#pragma unroll
            for (int i = 0; i < E; ++i) {
                md = fmaxf(md, fabsf(dov[i]));
                mv = fmaxf(mv, fabsf(bf2f(vs[i])));
            }
        }
    }
    if (p.gmax) {   // maxima of |dout| and |v|, one atomic each per workgroup
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) {
            md = fmaxf(md, __shfl_xor(md, m, 64));
            mv = fmaxf(mv, __shfl_xor(mv, m, 64));
        }
        if (lane == 0) { mx[0][wave] = md; mx[1][wave] = mv; }
        __syncthreads();
        if (threadIdx.x < 2) {
            const float* m4 = mx[threadIdx.x];
            atomicMax(p.gmax + threadIdx.x, __float_as_uint(fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3]))));
        }
    }
}

// Power-of-two scale of dS for its fp16 products: with m = max|dO| max|v|,
// |dS| <= |dO . v| + |D| <= 2 d m, so sigma = 2^-floor(log2 m) keeps sigma |dS|
// below 2 d while typical values stay in fp16's normal range (1 when m = 0).
__device__ __forceinline__ float ds_sigma(const unsigned* gmax) {
    const float m = __uint_as_float(gmax[0]) * __uint_as_float(gmax[1]);
    if (!(m > 0.f) || !(m < __builtin_huge_valf())) return 1.f;   // zero, inf or NaN: no scaling
    const int e = (int)((__float_as_uint(m) >> 23) & 0xffu) - 127;
    return ldexpf(1.f, -max(-100, min(e, 100)));
}

// ---------------------------------------------------------------------------------
// Shared epilogue: a wave's four 32x32 accumulators hold X^T for its 32 rows
// (lane n = row, element i of d-block db = column 32 db + 8(i/4) + 4h + i%4).
// Writes mul * X (+ add) to dst row `row` (fp32 or bf16).

__device__ __forceinline__ void store_rows(const f32x16 (&acc)[4], float mul, const float* add,
                                           const float* add2, void* dst, int out_f32,
                                           long long rowoff, int h) {
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int d0 = db * 32 + 8 * g + 4 * h;
            float r[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) r[i] = acc[db][4 * g + i] * mul;
            if (add) {
                const f32x4 x = *reinterpret_cast<const f32x4*>(add + rowoff + d0);
#pragma unroll
                for (int i = 0; i < 4; ++i) r[i] += x[i];
            }
            if (add2) {
                const f32x4 x = *reinterpret_cast<const f32x4*>(add2 + rowoff + d0);
#pragma unroll
                for (int i = 0; i < 4; ++i) r[i] += x[i];
            }
            if (out_f32) {
                *reinterpret_cast<f32x4*>(static_cast<float*>(dst) + rowoff + d0) =
                    f32x4{r[0], r[1], r[2], r[3]};
            } else {
                bf16x4 ov;
#pragma unroll
                for (int i = 0; i < 4; ++i) ov[i] = f2bf(r[i]);
                *reinterpret_cast<bf16x4*>(static_cast<bf16*>(dst) + rowoff + d0) = ov;
            }
        }
}

// Loads a wave's 32 rows of a [rows][128] bf16 tensor as MFMA B fragments
// (lane l: row l % 32, columns 16 ks + 8 (l / 32) .. +7); zero past the frame.
__device__ __forceinline__ void load_rows(bf16x8 (&f)[8], const bf16* p, bool valid, int h) {
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
        if (valid) f[ks] = *reinterpret_cast<const bf16x8*>(p + 16 * ks + 8 * h);
        else
#pragma unroll
            for (int j = 0; j < 8; ++j) f[ks][j] = (bf16)0.f;
    }
}

__device__ __forceinline__ void load_rows_h(f16x8 (&f)[8], const f16* p, bool valid, int h) {
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
        if (valid) f[ks] = *reinterpret_cast<const f16x8*>(p + 16 * ks + 8 * h);
        else
#pragma unroll
            for (int j = 0; j < 8; ++j) f[ks][j] = (f16)0.f;
    }
}

// ---------------------------------------------------------------------------------
// bf16 query pass: dq. One workgroup = 4 waves = 128 query rows of one frame.

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void win_bwd_dq_bf16_kernel(BwdLaunch w) {
    __shared__ __attribute__((aligned(1024))) char Kst[2][kTileB];
    __shared__ __attribute__((aligned(1024))) char Vst[2][kTileB];
    typedef __attribute__((address_space(3))) char lds_char;
    const uint32_t ldsK = (uint32_t)(uintptr_t)(lds_char*)&Kst[0][0];
    const uint32_t ldsV = (uint32_t)(uintptr_t)(lds_char*)&Vst[0][0];

    const int nqt = (w.P + kRows - 1) / kRows;
    const int nwg = w.BH * w.T * nqt;
    const int wid = xcd_remap(blockIdx.x, nwg);
    const int qt = wid % nqt;
    const int fq = w.T - 1 - (wid / nqt) % w.T;   // late frames (most taps) first
    const int bh = wid / (nqt * w.T);

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = lane & 31, h = lane >> 5;
    LaneOffs L;
    lane_offsets(L, wave, lane);

    // K staged in fp16 (for S and for dQ = K^T dS), V in bf16
    const bf16* kbh = static_cast<const bf16*>(w.k16) + (long long)bh * w.bh_elems;
    const bf16* vbh = static_cast<const bf16*>(w.v) + (long long)bh * w.bh_elems;
    const long long kv_frame = (long long)w.P * kD;

    const int nseg = taps_present(w.off, w.ntaps, fq);
    const int ntk = (w.P + kBK - 1) / kBK;
    const int nit = nseg * ntk;

    int isg = 0, itk = 0;   // next tile to stage
    auto issue = [&](uint32_t stage) {
        const long long ofs = (long long)(fq - w.off[isg]) * kv_frame + (long long)itk * kBK * kD;
        issue_tile(ldsK + stage * kTileB, ldsV + stage * kTileB, kbh + ofs, vbh + ofs,
                   min(kBK, w.P - itk * kBK), wave, lane, L);
        if (++itk == ntk) { itk = 0; ++isg; }
    };
    if (nit > 0) issue(0);

    const int qrow = qt * kRows + wave * 32 + n;
    const bool valid = qrow < w.P;
    const bool wave_rows = qt * kRows + wave * 32 < w.P;
    const long long rowoff = (long long)bh * w.bh_elems + ((long long)fq * w.P + qrow) * kD;
    f16x8 qf[8];
    bf16x8 df[8];
    load_rows_h(qf, static_cast<const f16*>(w.q16) + rowoff, valid, h);
    load_rows(df, static_cast<const bf16*>(w.dout) + rowoff, valid, h);
    const long long srow = (long long)bh * w.T * w.P + (long long)fq * w.P + qrow;
    const float lse2 = valid ? w.stats[2 * srow] : 0.f;
    const float Dq = valid ? w.stats[2 * srow + 1] : 0.f;
    const int eq = qk_exp(w.gmax[2]), ek = qk_exp(w.gmax[3]);
    const float c = ldexpf(w.scale * kLog2e, -(eq + ek));   // the logits come from 2^eq q, 2^ek k
    const float sig = ds_sigma(w.gmax);

    f32x16 acc[4];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[db][i] = 0.f;

    int tk = 0;   // tile being consumed (within its segment)
    auto step = [&](int it, auto stage_tag) {
        constexpr int ST = decltype(stage_tag)::value;
        wait_vmcnt<0>();
        __syncthreads();
        if (it + 1 < nit) issue(ST ^ 1);
        const int nvalid = min(kBK, w.P - tk * kBK);
        if (wave_rows) {
            const char* Ks = Kst[ST];
            const char* Vs = Vst[ST];
            // one 32-key block at a time keeps the live logits to 32 registers
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                f32x16 s, dp;
                const f32x16 zero = {};
#pragma unroll
                for (int ks = 0; ks < 8; ++ks) {
                    const f16x8 kf = *reinterpret_cast<const f16x8*>(Ks + kb * 32 * kRowB + L.k[ks]);
                    s = mfma32h(kf, qf[ks], ks == 0 ? zero : s);
                    const bf16x8 vf = *reinterpret_cast<const bf16x8*>(Vs + kb * 32 * kRowB + L.k[ks]);
                    dp = mfma32(vf, df[ks], ks == 0 ? zero : dp);
                }
                // sigma ds in fp16 (11 significant bits)
                f16x8 dsf[2];
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int key = kb * 32 + 8 * (i >> 2) + 4 * h + (i & 3);
                    const float p = fast_exp2(__builtin_fmaf(s[i], c, -lse2));
                    const float ds = key < nvalid ? (p * sig) * (dp[i] - Dq) : 0.f;
                    dsf[i >> 3][i & 7] = (f16)ds;
                }
#pragma unroll
                for (int gg = 0; gg < 2; ++gg)
#pragma unroll
                    for (int db = 0; db < 4; ++db) {
                        const char* kb_ = Ks + (kb * 32 + 16 * gg) * kRowB;
                        const f16x4 lo = tr_f16(kb_ + L.v[db]);
                        const f16x4 hi = tr_f16(kb_ + L.vh[db]);
                        acc[db] = mfma32h(cat(lo, hi), dsf[gg], acc[db]);
                    }
            }
        }
        if (++tk == ntk) tk = 0;
    };
    for (int it = 0; it < nit; it += 2) {
        step(it, std::integral_constant<int, 0>{});
        if (it + 1 < nit) step(it + 1, std::integral_constant<int, 1>{});
    }
    if (!valid) return;
    store_rows(acc, ldexpf(w.scale / sig, -ek), w.add_q, w.add2_q, w.dq, w.out_f32, rowoff, h);
}

// ---------------------------------------------------------------------------------
// bf16 key pass: one workgroup = 4 waves = 128 keys of one key frame, walking the
// query tiles (Q, dO and their stats, staged in LDS) of every frame whose window
// holds that key frame. Two launches of the same kernel: DK accumulates dK^T
// (needs S, dP and dS), the other dV^T (needs S and P); keeping one accumulator
// set per launch keeps each within 256 registers at two waves per SIMD, at the
// price of computing S twice.

template <bool DK>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void win_bwd_key_bf16_kernel(BwdLaunch w) {
    __shared__ __attribute__((aligned(1024))) char Qst[2][kTileB];
    __shared__ __attribute__((aligned(1024))) char Ost[2][kTileB];
    __shared__ __attribute__((aligned(16))) float Sst[2][2 * kBK];   // {lse2, D} per query
    typedef __attribute__((address_space(3))) char lds_char;
    const uint32_t ldsQ = (uint32_t)(uintptr_t)(lds_char*)&Qst[0][0];
    const uint32_t ldsO = (uint32_t)(uintptr_t)(lds_char*)&Ost[0][0];
    const uint32_t ldsS = (uint32_t)(uintptr_t)(lds_char*)&Sst[0][0];

    const int nkt = (w.P + kRows - 1) / kRows;
    const int nwg = w.BH * w.T * nkt;
    const int wid = xcd_remap(blockIdx.x, nwg);
    const int kt = wid % nkt;
    const int fk = (wid / nkt) % w.T;   // early key frames (most attending frames) first
    const int bh = wid / (nkt * w.T);

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = lane & 31, h = lane >> 5;
    LaneOffs L;
    lane_offsets(L, wave, lane);

    // Q staged in fp16 (for S and for dK = Q^T dS), dO in bf16
    const bf16* qbh = static_cast<const bf16*>(w.q16) + (long long)bh * w.bh_elems;
    const bf16* obh = static_cast<const bf16*>(w.dout) + (long long)bh * w.bh_elems;
    const float* sbh = w.stats + 2 * (long long)bh * w.T * w.P;

    // attending query frames fk + off[j] < T: a prefix of the ascending offsets
    int nseg = 0;
    for (int j = 0; j < w.ntaps; ++j) nseg += (fk + w.off[j] < w.T) ? 1 : 0;
    const int ntq = (w.P + kBK - 1) / kBK;
    const int nit = nseg * ntq;

    int isg = 0, itq = 0;   // next tile to stage
    auto issue = [&](uint32_t stage) {
        const long long r0 = (long long)(fk + w.off[isg]) * w.P + (long long)itq * kBK;
        issue_tile(ldsQ + stage * kTileB, ldsO + stage * kTileB, qbh + r0 * kD, obh + r0 * kD,
                   min(kBK, w.P - itq * kBK), wave, lane, L);
        // stats of the tile's 64 queries (512 bytes, two dword loads); rows past the
        // frame read on into the next rows or the 64-row padding, never used
        if (wave == 0) {
            dma4((uint32_t)lane * 4u, sbh + 2 * r0, ldsS + stage * 512u);
            dma4((uint32_t)lane * 4u + 256u, sbh + 2 * r0, ldsS + stage * 512u + 256u);
        }
        if (++itq == ntq) { itq = 0; ++isg; }
    };
    if (nit > 0) issue(0);

    const int krow = kt * kRows + wave * 32 + n;
    const bool valid = krow < w.P;
    const bool wave_rows = kt * kRows + wave * 32 < w.P;
    const long long rowoff = (long long)bh * w.bh_elems + ((long long)fk * w.P + krow) * kD;
    f16x8 kf[8];
    bf16x8 vf[DK ? 8 : 1];
    load_rows_h(kf, static_cast<const f16*>(w.k16) + rowoff, valid, h);
    if (DK) load_rows(reinterpret_cast<bf16x8(&)[8]>(vf), static_cast<const bf16*>(w.v) + rowoff, valid, h);
    const int eq = qk_exp(w.gmax[2]), ek = qk_exp(w.gmax[3]);
    const float c = ldexpf(w.scale * kLog2e, -(eq + ek));   // the logits come from 2^eq q, 2^ek k
    const float sig = ds_sigma(w.gmax);

    f32x16 acc[4];   // dK^T or dV^T
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[db][i] = 0.f;

    int tq = 0;   // tile being consumed (within its segment)
    auto step = [&](int it, auto stage_tag) {
        constexpr int ST = decltype(stage_tag)::value;
        wait_vmcnt<0>();
        __syncthreads();
        if (it + 1 < nit) issue(ST ^ 1);
        const int nvalid = min(kBK, w.P - tq * kBK);
        if (wave_rows) {
            const char* Qs = Qst[ST];
            const char* Os = Ost[ST];
            const float* Ss = Sst[ST];
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                f32x16 s, dp;
                const f32x16 zero = {};
#pragma unroll
                for (int ks = 0; ks < 8; ++ks) {
                    const f16x8 qa = *reinterpret_cast<const f16x8*>(Qs + qb * 32 * kRowB + L.k[ks]);
                    s = mfma32h(qa, kf[ks], ks == 0 ? zero : s);
                    if (DK) {
                        const bf16x8 oa = *reinterpret_cast<const bf16x8*>(Os + qb * 32 * kRowB + L.k[ks]);
                        dp = mfma32(oa, vf[DK ? ks : 0], ks == 0 ? zero : dp);
                    }
                }
                // element i: query qb*32 + 8(i/4) + 4h + i%4 of the tile, key n
                f16x8 dsf[2];   // DK: sigma dS in fp16
                bf16x8 pf[2];   // dV: P in bf16
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int q0 = qb * 32 + 8 * g + 4 * h;
                    const f32x4 st0 = *reinterpret_cast<const f32x4*>(Ss + 2 * q0);
                    const f32x4 st1 = *reinterpret_cast<const f32x4*>(Ss + 2 * q0 + 4);
                    const float l2[4] = {st0[0], st0[2], st1[0], st1[2]};
                    const float dd[4] = {st0[1], st0[3], st1[1], st1[3]};
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int i = 4 * g + r;
                        const bool ok = q0 + r < nvalid;
                        const float p = fast_exp2(__builtin_fmaf(s[i], c, -l2[r]));
                        if (DK) dsf[i >> 3][i & 7] = (f16)(ok ? (p * sig) * (dp[i] - dd[r]) : 0.f);
                        else pf[i >> 3][i & 7] = f2bf(ok ? p : 0.f);
                    }
                }
#pragma unroll
                for (int gg = 0; gg < 2; ++gg)
#pragma unroll
                    for (int db = 0; db < 4; ++db) {
                        if (DK) {   // dK^T += Q^T dS
                            const char* b_ = Qs + (qb * 32 + 16 * gg) * kRowB;
                            acc[db] = mfma32h(cat(tr_f16(b_ + L.v[db]), tr_f16(b_ + L.vh[db])),
                                              dsf[gg], acc[db]);
                        } else {    // dV^T += dO^T P
                            const char* b_ = Os + (qb * 32 + 16 * gg) * kRowB;
                            acc[db] = mfma32(cat(tr_bf16(b_ + L.v[db]), tr_bf16(b_ + L.vh[db])),
                                             pf[gg], acc[db]);
                        }
                    }
            }
        }
        if (++tq == ntq) tq = 0;
    };
    for (int it = 0; it < nit; it += 2) {
        step(it, std::integral_constant<int, 0>{});
        if (it + 1 < nit) step(it + 1, std::integral_constant<int, 1>{});
    }
    if (!valid) return;
    if (DK) store_rows(acc, ldexpf(w.scale / sig, -eq), w.add_k, w.add2_k, w.dk, w.out_f32, rowoff, h);
    else store_rows(acc, 1.f, w.add_v, w.add2_v, w.dv, w.out_f32, rowoff, h);
}

// ---------------------------------------------------------------------------------
// fp32 passes (d = 64 or 128): 64 rows per workgroup, 4 lanes per row, each lane
// owning d/4 interleaved columns; the other side is read from global memory.

template <int D>
__device__ __forceinline__ float dot4(const float (&a)[D / 4], const float* b, int sub) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < D / 4; ++i) s = __builtin_fmaf(a[i], b[4 * i + sub], s);
    s += __shfl_xor(s, 1, 64);
    s += __shfl_xor(s, 2, 64);
    return s;
}

template <int D>
__global__ __launch_bounds__(256) void win_bwd_dq_f32_kernel(BwdLaunch w) {
    const int nqt = (w.P + 63) / 64;
    const int wid = blockIdx.x;
    const int qt = wid % nqt;
    const int fq = (wid / nqt) % w.T;
    const int bh = wid / (nqt * w.T);
    const int sub = threadIdx.x & 3;
    const int row = qt * 64 + (threadIdx.x >> 2);
    const bool valid = row < w.P;
    const int prow = valid ? row : w.P - 1;   // duplicates of the last row, never stored
    const long long rowoff = (long long)bh * w.bh_elems + ((long long)fq * w.P + prow) * D;
    const float* kbh = static_cast<const float*>(w.k) + (long long)bh * w.bh_elems;
    const float* vbh = static_cast<const float*>(w.v) + (long long)bh * w.bh_elems;
    float qv[D / 4], dov[D / 4], acc[D / 4];
#pragma unroll
    for (int i = 0; i < D / 4; ++i) {
        qv[i] = static_cast<const float*>(w.q)[rowoff + 4 * i + sub];
        dov[i] = static_cast<const float*>(w.dout)[rowoff + 4 * i + sub];
        acc[i] = 0.f;
    }
    const long long srow = (long long)bh * w.T * w.P + (long long)fq * w.P + prow;
    const float lse2 = w.stats[2 * srow], Dq = w.stats[2 * srow + 1];
    const float c = w.scale * kLog2e;
    const int nseg = taps_present(w.off, w.ntaps, fq);
    for (int sg = 0; sg < nseg; ++sg) {
        const long long f0 = (long long)(fq - w.off[sg]) * w.P * D;
        for (int p = 0; p < w.P; ++p) {
            const float* kr = kbh + f0 + (long long)p * D;
            const float* vr = vbh + f0 + (long long)p * D;
            const float z = dot4<D>(qv, kr, sub);
            const float dp = dot4<D>(dov, vr, sub);
            const float ds = exp2f(__builtin_fmaf(z, c, -lse2)) * (dp - Dq);
#pragma unroll
            for (int i = 0; i < D / 4; ++i) acc[i] = __builtin_fmaf(ds, kr[4 * i + sub], acc[i]);
        }
    }
    if (!valid) return;
#pragma unroll
    for (int i = 0; i < D / 4; ++i) {
        float r = acc[i] * w.scale;
        if (w.add_q) r += w.add_q[rowoff + 4 * i + sub];
        if (w.add2_q) r += w.add2_q[rowoff + 4 * i + sub];
        static_cast<float*>(w.dq)[rowoff + 4 * i + sub] = r;
    }
}

template <int D>
__global__ __launch_bounds__(256) void win_bwd_dkdv_f32_kernel(BwdLaunch w) {
    const int nkt = (w.P + 63) / 64;
    const int wid = blockIdx.x;
    const int kt = wid % nkt;
    const int fk = (wid / nkt) % w.T;
    const int bh = wid / (nkt * w.T);
    const int sub = threadIdx.x & 3;
    const int row = kt * 64 + (threadIdx.x >> 2);
    const bool valid = row < w.P;
    const int prow = valid ? row : w.P - 1;
    const long long rowoff = (long long)bh * w.bh_elems + ((long long)fk * w.P + prow) * D;
    const float* qbh = static_cast<const float*>(w.q) + (long long)bh * w.bh_elems;
    const float* obh = static_cast<const float*>(w.dout) + (long long)bh * w.bh_elems;
    const float* sbh = w.stats + 2 * (long long)bh * w.T * w.P;
    float kv[D / 4], vv[D / 4], dk[D / 4], dv[D / 4];
#pragma unroll
    for (int i = 0; i < D / 4; ++i) {
        kv[i] = static_cast<const float*>(w.k)[rowoff + 4 * i + sub];
        vv[i] = static_cast<const float*>(w.v)[rowoff + 4 * i + sub];
        dk[i] = 0.f;
        dv[i] = 0.f;
    }
    const float c = w.scale * kLog2e;
    for (int j = 0; j < w.ntaps; ++j) {
        const int fq = fk + w.off[j];
        if (fq >= w.T) break;
        for (int p = 0; p < w.P; ++p) {
            const long long t = (long long)fq * w.P + p;
            const float* qr = qbh + t * D;
            const float* dr = obh + t * D;
            const float z = dot4<D>(kv, qr, sub);
            const float dp = dot4<D>(vv, dr, sub);
            const float pr = exp2f(__builtin_fmaf(z, c, -sbh[2 * t]));
            const float ds = pr * (dp - sbh[2 * t + 1]);
#pragma unroll
            for (int i = 0; i < D / 4; ++i) {
                dk[i] = __builtin_fmaf(ds, qr[4 * i + sub], dk[i]);
                dv[i] = __builtin_fmaf(pr, dr[4 * i + sub], dv[i]);
            }
        }
    }
    if (!valid) return;
#pragma unroll
    for (int i = 0; i < D / 4; ++i) {
        float a = dk[i] * w.scale, b = dv[i];
        if (w.add_k) a += w.add_k[rowoff + 4 * i + sub];
        if (w.add_v) b += w.add_v[rowoff + 4 * i + sub];
        if (w.add2_k) a += w.add2_k[rowoff + 4 * i + sub];
        if (w.add2_v) b += w.add2_v[rowoff + 4 * i + sub];
        static_cast<float*>(w.dk)[rowoff + 4 * i + sub] = a;
        static_cast<float*>(w.dv)[rowoff + 4 * i + sub] = b;
    }
}

}  // namespace

hipError_t launch_win_bwd_prep(const BwdPrep& p, hipStream_t stream) {
    if (p.rows == 0) return hipSuccess;
    if (p.q16) {   // the copies' scales first (gmax[2], gmax[3], zeroed by the caller)
        if (p.d != 128 || !p.gmax) return hipErrorInvalidValue;
        const long long n8 = p.rows * 128 / 8;
        const long long g = std::min((n8 + 255) / 256, 2048LL);
        hipLaunchKernelGGL(win_bwd_qkmax_kernel, dim3((unsigned)g), dim3(256), 0, stream,
                           static_cast<const bf16*>(p.q), static_cast<const bf16*>(p.k), n8, p.gmax);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const long long nwg = std::min((p.rows + 15) / 16, 4096LL);
    if (p.d == 128)
        hipLaunchKernelGGL((win_bwd_prep_kernel<128>), dim3((unsigned)nwg), dim3(256), 0, stream, p);
    else if (p.d == 64)
        hipLaunchKernelGGL((win_bwd_prep_kernel<64>), dim3((unsigned)nwg), dim3(256), 0, stream, p);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_win_bwd(const BwdLaunch& b, hipStream_t stream, int parts) {
    if (b.BH == 0 || b.T == 0 || b.P == 0) return hipSuccess;
    if (b.dtype == 1) {   // bf16, d == 128
        const long long nwg = (long long)b.BH * b.T * ((b.P + kRows - 1) / kRows);
        if (nwg > 0x7fffffffLL) return hipErrorInvalidValue;
        if (parts & kBwdQuery)
            hipLaunchKernelGGL(win_bwd_dq_bf16_kernel, dim3((unsigned)nwg), dim3(256), 0, stream, b);
        if (parts & kBwdKey) {
            hipLaunchKernelGGL(win_bwd_key_bf16_kernel<true>, dim3((unsigned)nwg), dim3(256), 0, stream, b);
            hipLaunchKernelGGL(win_bwd_key_bf16_kernel<false>, dim3((unsigned)nwg), dim3(256), 0, stream, b);
        }
        return hipGetLastError();
    }
    const long long nwg = (long long)b.BH * b.T * ((b.P + 63) / 64);
    if (nwg > 0x7fffffffLL) return hipErrorInvalidValue;
    const dim3 g((unsigned)nwg), blk(256);
    if (b.d == 64) {
        if (parts & kBwdQuery) hipLaunchKernelGGL((win_bwd_dq_f32_kernel<64>), g, blk, 0, stream, b);
        if (parts & kBwdKey) hipLaunchKernelGGL((win_bwd_dkdv_f32_kernel<64>), g, blk, 0, stream, b);
    } else {
        if (parts & kBwdQuery) hipLaunchKernelGGL((win_bwd_dq_f32_kernel<128>), g, blk, 0, stream, b);
        if (parts & kBwdKey) hipLaunchKernelGGL((win_bwd_dkdv_f32_kernel<128>), g, blk, 0, stream, b);
    }
    return hipGetLastError();
}

}  // namespace hta
