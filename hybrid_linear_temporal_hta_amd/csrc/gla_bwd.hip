// gla_bwd.hip -- backward pass of the gated-delta GLA branch.
//
// Forward (page "Kairos：面向物理 AI 的原生世界模型栈" (yingwang.github.io), section
// 二、方法, GLA paragraph and update equations), with the state kept as M = S^T
// (dk x dv) and u_t = M_{t-1}^T k_t:
//   form 0 (GatedDeltaNet reading): M_t = alpha_t M_{t-1} - alpha_t beta_t k_t u_t^T + beta_t k_t v_t^T
//   form 1 (the printed update):    M_t = alpha_t M_{t-1} -         beta_t k_t u_t^T + beta_t k_t v_t^T
//   o_t = scale M_t^T q_t.
// The backward is the chain rule through this recurrence, run in reverse with
// the state's adjoint G_t = dL/dM_t:
//   G += scale q_t dO_t^T;  dq_t = scale M_t dO_t;  w = G^T k_t;  dv_t = beta_t w
//   form 0: dalpha_t = <G, M_{t-1} - beta k u^T>, dbeta_t = w.(v - alpha u),
//           du = -alpha beta w, dk_t = beta G (v - alpha u) + M_{t-1} du
//   form 1: dalpha_t = <G, M_{t-1}>, dbeta_t = w.(v - u),
//           du = -beta w,       dk_t = beta G (v - u) + M_{t-1} du
//   G <- alpha_t G + k_t du^T.
//
// fp32 path (small workloads): one workgroup per (b, h) runs exactly this, token
// by token, with the forward states recomputed from checkpoints every 64 tokens
// (the checkpoints and one segment of states live in the workspace).
//
// bf16 path: the chunked (UT / WY) form of the forward, differentiated chunk by
// chunk. Per chunk of C = 64 tokens entering with M0 (notation of the forward
// kernels: g the inclusive cumulative sum of log alpha in the chunk, gp = g or
// its exclusive version for the printed form, E = e^g, Dn = e^{g_C - g},
// Ep = e^{gp}, T = (I + A)^-1, Pm = tril(Q K^T o e^{g_i - g_j})):
//   R = diag(beta) (V - diag(Ep) K M0),  U = T R,
//   O = scale (diag(E) Q M0 + Pm U),  M_C = E_C M0 + K^T diag(Dn) U.
// With Gb = scale dO and dM_C = dL/dM_C:
//   dU = Pm^T Gb + diag(Dn) K dM_C,  dR = T^T dU,
//   dM0 = E_C dM_C + Q^T diag(E) Gb - K^T diag(beta Ep) dR      (the reverse scan),
// and, per chunk once dR and dM_C are known (the gradient kernel),
//   dQ = diag(E) Gb M0^T + D1 K,              D1 = (Gb U^T) o tril(e^{g_i - g_j})
//   dK = D1^T Q + diag(Dn) U dM_C^T - diag(beta Ep) dR M0^T + (Bm + Bm^T) K,
//        dA = -strictly-lower(dR U^T),  Bm = diag(beta) (dA o e^{gp_i - g_j})
//   dV = diag(beta) dR
//   dbeta_i = dR_i.V_i - Ep_i K_i.(dR M0^T)_i + sum_j (dA o e^{gp_i - g_j} o K K^T)_ij
//   and dg, dgp (then dlog alpha = reverse cumulative sums) from every place g
//   and gp enter: E in O, Pm, A, Ep in R, and M_C.
// Six launches: the forward prep and scan (saving each chunk's M0 and U in
// fp16); a pass taking max |scale dO| and max |dL/dM_L|, and one scaling
// scale * dO into fp16 by the power of two taken from them (so the fp16 operands
// keep their precision whatever the gradient's magnitude; the results are scaled
// back exactly); the reverse scan (one workgroup per (b, h, 64 value columns),
// chunks in reverse order, dM in fp32 registers; it saves dM_C and dR per chunk
// in fp16); and the chunk-parallel gradient kernel (one workgroup per chunk).
#include <string.h>

#include <type_traits>

#include "device_common.h"
#include "gla_tiles.h"
#include "hta_internal.h"

namespace hta {

namespace {

using namespace glat;

constexpr int kCk = 64;                // tokens per checkpoint segment (fp32 path)

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    return v;
}

// ---------------------------------------------------------------------------------
// fp32 token-level kernel. Thread t owns column j = t % D of M and G, rows
// i = rg + R r (rg = t / D, R = 256 / D row groups, r < D / R).

template <int D>
__global__ __launch_bounds__(256) void gla_bwd_f32_kernel(GlaBwdLaunch b) {
    constexpr int R = 256 / D;
    constexpr int NR = D / R;
    __shared__ float qs[D], ks[D], vs[D], gs_[D];   // token vectors (gs_ = dO)
    __shared__ float part[R][D];                   // column-sum partials
    __shared__ float rowp[4][NR];                  // row-sum partials per wave
    __shared__ float red[4];
    __shared__ float usum[D], wsum[D];

    const int bh = blockIdx.x, t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int j = t % D, rg = t / D;
    const long long L = b.L;
    const long long DD = (long long)D * D;
    const long long nck = (L + kCk - 1) / kCk;
    float* ckpt = static_cast<float*>(b.ws) + (long long)bh * (nck + 1) * DD;
    float* seg = static_cast<float*>(b.ws) + (long long)b.BH * (nck + 1) * DD +
                 (long long)bh * (kCk + 1) * DD;
    const float* q = static_cast<const float*>(b.q) + (long long)bh * L * D;
    const float* k = static_cast<const float*>(b.k) + (long long)bh * L * D;
    const float* v = static_cast<const float*>(b.v) + (long long)bh * L * D;
    const float* dO = static_cast<const float*>(b.dout) + (long long)bh * L * D;
    const float* al = b.alpha + (long long)bh * L;
    const float* be = b.beta + (long long)bh * L;
    float* dq = static_cast<float*>(b.dq) + (long long)bh * L * D;
    float* dk = static_cast<float*>(b.dk) + (long long)bh * L * D;
    float* dv = static_cast<float*>(b.dv) + (long long)bh * L * D;
    float* st = b.dstate + (long long)bh * DD;
    const float* s0 = b.state0 + (long long)bh * DD;
    auto idx = [&](int r) { return (long long)(rg + R * r) * D + j; };

    // one forward token step on M (ks, vs staged); u is left in usum
    auto fwd_step = [&](float (&M)[NR], float a, float bt) {
        float p = 0.f;
#pragma unroll
        for (int r = 0; r < NR; ++r) p += M[r] * ks[rg + R * r];
        part[rg][j] = p;
        __syncthreads();
        float u = 0.f;
#pragma unroll
        for (int g = 0; g < R; ++g) u += part[g][j];
        const float ea = b.form == 0 ? a * bt : bt;
        const float vj = vs[j];
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            const float ki = ks[rg + R * r];
            M[r] = a * M[r] - ea * ki * u + bt * ki * vj;
        }
    };
    auto stage_kv = [&](long long tt) {
        for (int e = t; e < 2 * D; e += 256) {
            if (e < D) ks[e] = k[tt * D + e];
            else vs[e - D] = v[tt * D + e - D];
        }
    };

    // forward pass: checkpoints M_0, M_64, ...
    float M[NR], G[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) { M[r] = s0[idx(r)]; ckpt[idx(r)] = M[r]; }
    for (long long tt = 0; tt < L; ++tt) {
        __syncthreads();
        stage_kv(tt);
        __syncthreads();
        fwd_step(M, al[tt], be[tt]);
        if ((tt + 1) % kCk == 0) {
#pragma unroll
            for (int r = 0; r < NR; ++r) ckpt[((tt + 1) / kCk) * DD + idx(r)] = M[r];
        }
    }

    // reverse pass
#pragma unroll
    for (int r = 0; r < NR; ++r) G[r] = st[idx(r)];
    const float sc = b.scale;
    for (long long c = nck - 1; c >= 0; --c) {
        const long long t0 = c * kCk, t1 = min(t0 + kCk, L);
#pragma unroll
        for (int r = 0; r < NR; ++r) { M[r] = ckpt[c * DD + idx(r)]; seg[idx(r)] = M[r]; }
        for (long long tt = t0; tt < t1; ++tt) {
            __syncthreads();
            stage_kv(tt);
            __syncthreads();
            fwd_step(M, al[tt], be[tt]);
#pragma unroll
            for (int r = 0; r < NR; ++r) seg[(tt - t0 + 1) * DD + idx(r)] = M[r];
        }
        for (long long tt = t1 - 1; tt >= t0; --tt) {
            __syncthreads();
            for (int e = t; e < 4 * D; e += 256) {
                const int w = e / D, x = e % D;
                if (w == 0) qs[x] = q[tt * D + x];
                else if (w == 1) ks[x] = k[tt * D + x];
                else if (w == 2) vs[x] = v[tt * D + x];
                else gs_[x] = dO[tt * D + x];
            }
            __syncthreads();
            const float a = al[tt], bt = be[tt];
            const float doj = gs_[j];
            // G += scale q dO^T; dq = scale M_t dO (row sums)
#pragma unroll
            for (int r = 0; r < NR; ++r) {
                G[r] += sc * qs[rg + R * r] * doj;
                const float x = wave_sum(seg[(tt - t0 + 1) * DD + idx(r)] * doj);
                if (lane == 0) rowp[wave][r] = x;
            }
            float Mp[NR];
#pragma unroll
            for (int r = 0; r < NR; ++r) Mp[r] = seg[(tt - t0) * DD + idx(r)];
            // w = G^T k, u = M_{t-1}^T k (column sums)
            {
                float pw = 0.f, pu = 0.f;
#pragma unroll
                for (int r = 0; r < NR; ++r) {
                    pw += G[r] * ks[rg + R * r];
                    pu += Mp[r] * ks[rg + R * r];
                }
                part[rg][j] = pw;
                __syncthreads();
                if (t < D) {
                    float s = 0.f;
                    for (int g = 0; g < R; ++g) s += part[g][t];
                    wsum[t] = s;
                }
                if (t < D) {   // dq row t
                    const int rr = t / R, g0 = t % R;
                    float s = 0.f;
                    for (int w = 0; w < 4; ++w)
                        if ((w * 64) / D == g0) s += rowp[w][rr];
                    dq[tt * D + t] = sc * s;
                }
                __syncthreads();
                part[rg][j] = pu;
                __syncthreads();
                if (t < D) {
                    float s = 0.f;
                    for (int g = 0; g < R; ++g) s += part[g][t];
                    usum[t] = s;
                }
                __syncthreads();
            }
            const float ua = b.form == 0 ? a : 1.f;
            const float wj = wsum[j], uj = usum[j];
            const float duj = -ua * bt * wj;
            // dalpha (all elements), dbeta (each column once), dk (row sums)
            float pa = 0.f;
#pragma unroll
            for (int r = 0; r < NR; ++r) {
                const float ki = ks[rg + R * r];
                const float erase = b.form == 0 ? bt * ki * uj : 0.f;
                pa += G[r] * (Mp[r] - erase);
                const float x = wave_sum(G[r] * bt * (vs[j] - ua * uj) + Mp[r] * duj);
                if (lane == 0) rowp[wave][r] = x;
            }
            pa = wave_sum(pa);
            float pb = (rg == 0) ? wj * (vs[j] - ua * uj) : 0.f;
            pb = wave_sum(pb);
            if (lane == 0) red[wave] = pa;
            __syncthreads();
            if (t < D) {
                const int rr = t / R, g0 = t % R;
                float s = 0.f;
                for (int w = 0; w < 4; ++w)
                    if ((w * 64) / D == g0) s += rowp[w][rr];
                dk[tt * D + t] = s;
                dv[tt * D + t] = bt * wsum[t];
            }
            if (t == 0) b.dalpha[(long long)bh * L + tt] = red[0] + red[1] + red[2] + red[3];
            __syncthreads();
            if (lane == 0) red[wave] = pb;
            __syncthreads();
            if (t == 0) b.dbeta[(long long)bh * L + tt] = red[0] + red[1] + red[2] + red[3];
            // G <- alpha G + k du^T
#pragma unroll
            for (int r = 0; r < NR; ++r) G[r] = a * G[r] + ks[rg + R * r] * duj;
        }
    }
#pragma unroll
    for (int r = 0; r < NR; ++r) st[idx(r)] = G[r];
}

// ---------------------------------------------------------------------------------
// bf16 path: workspace regions.

constexpr size_t kAl = 256;
__host__ __device__ inline size_t al256(size_t x) { return (x + kAl - 1) / kAl * kAl; }

struct BwdWs {
    unsigned* maxbits;   // float bits: [0] max |scale dO|, |dL/dM_L|; [1] max |v|, |M_0|
    float* state;        // copy of the initial state (the forward scan runs in place)
    char* blocks;        // chunk operand blocks of the forward prep
    f16* save_m;         // [BH][nch][128][128] M0 per chunk
    f16* save_u;         // [BH][nch][64][128] U per chunk
    f16* dme;            // [BH][nch][128][128] dL/dM_C per chunk (scaled)
    f16* dr;             // [BH][nch][64][128] dR per chunk (scaled)
    f16* gh;             // [BH][L][128] sigma * scale * dO
};

__host__ __device__ inline BwdWs bwd_ws(void* base, int BH, long long L) {
    const long long nch = (L + kC - 1) / kC;
    char* p = static_cast<char*>(base);
    BwdWs w;
    w.maxbits = reinterpret_cast<unsigned*>(p); p += kAl;
    w.state = reinterpret_cast<float*>(p); p += al256((size_t)BH * kD * kD * 4);
    w.blocks = p; p += al256((size_t)BH * nch * kChunkBytes);
    w.save_m = reinterpret_cast<f16*>(p); p += al256((size_t)BH * nch * kD * kD * 2);
    w.save_u = reinterpret_cast<f16*>(p); p += al256((size_t)BH * nch * kC * kD * 2);
    w.dme = reinterpret_cast<f16*>(p); p += al256((size_t)BH * nch * kD * kD * 2);
    w.dr = reinterpret_cast<f16*>(p); p += al256((size_t)BH * nch * kC * kD * 2);
    w.gh = reinterpret_cast<f16*>(p); p += al256((size_t)BH * L * kD * 2);
    return w;
}
inline size_t bwd_ws_bytes(int BH, long long L) {
    const long long nch = (L + kC - 1) / kC;
    return kAl + al256((size_t)BH * kD * kD * 4) + al256((size_t)BH * nch * kChunkBytes) +
           2 * al256((size_t)BH * nch * kD * kD * 2) + 2 * al256((size_t)BH * nch * kC * kD * 2) +
           al256((size_t)BH * L * kD * 2);
}

// maxbits[0] = max(|scale dO|, |dL/dM_L|) and maxbits[1] = max(|v|, |M_0|) (atomic
// max on the bits of non-negative floats). dO and v are read 16 bytes per lane,
// four loads in flight per thread; |scale| is applied to the maximum (rounding is
// monotonic: the same value as the maximum of the rounded products).
__global__ __launch_bounds__(256) void gla_bwd_max_kernel(GlaBwdLaunch b, unsigned* maxbits) {
    const long long nd = (long long)b.BH * b.L * kD, ns = (long long)b.BH * kD * kD;
    const long long stride = (long long)gridDim.x * 256;
    const long long t = (long long)blockIdx.x * 256 + threadIdx.x;
    float m = 0.f, mv = 0.f;
    {
        const long long n8 = nd / 8;
        const bf16x8* p = static_cast<const bf16x8*>(b.v);
        for (long long e = t; e < n8; e += 4 * stride) {
            bf16x8 x[4];
#pragma unroll
            for (int u = 0; u < 4; ++u)
                if (e + u * stride < n8) x[u] = p[e + u * stride];
#pragma unroll
            for (int u = 0; u < 4; ++u)
                if (e + u * stride < n8)
#pragma unroll
                    for (int i = 0; i < 8; ++i) mv = fmaxf(mv, fabsf(bf2f(x[u][i])));
        }
        for (long long e = t; e < ns; e += stride) mv = fmaxf(mv, fabsf(b.state0[e]));
    }
    if (b.do_f32) {
        const long long n4 = nd / 4;
        const f32x4* p = static_cast<const f32x4*>(b.dout);
        for (long long e = t; e < n4; e += 4 * stride) {
            f32x4 x[4];
#pragma unroll
            for (int u = 0; u < 4; ++u)
                x[u] = e + u * stride < n4 ? p[e + u * stride] : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int i = 0; i < 4; ++i) m = fmaxf(m, fabsf(x[u][i]));
        }
    } else {
        const long long n8 = nd / 8;
        const bf16x8* p = static_cast<const bf16x8*>(b.dout);
        for (long long e = t; e < n8; e += 4 * stride) {
            bf16x8 x[4];
#pragma unroll
            for (int u = 0; u < 4; ++u)
                if (e + u * stride < n8) x[u] = p[e + u * stride];
#pragma unroll
            for (int u = 0; u < 4; ++u)
                if (e + u * stride < n8)
#pragma unroll
                    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(bf2f(x[u][i])));
        }
    }
    m *= fabsf(b.scale);
    for (long long e = t; e < ns; e += stride) m = fmaxf(m, fabsf(b.dstate[e]));
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) {
        m = fmaxf(m, __shfl_xor(m, s, 64));
        mv = fmaxf(mv, __shfl_xor(mv, s, 64));
    }
    __shared__ float wm[2][4];   // one atomic per workgroup: same-address atomics serialise
    if ((threadIdx.x & 63) == 0) {
        wm[0][threadIdx.x >> 6] = m;
        wm[1][threadIdx.x >> 6] = mv;
    }
    __syncthreads();
    if (threadIdx.x < 2) {
        const float* r = wm[threadIdx.x];
        atomicMax(maxbits + threadIdx.x, __float_as_uint(fmaxf(fmaxf(r[0], r[1]), fmaxf(r[2], r[3]))));
    }
}

// gh = fp16(sigma * scale * dO), 8 elements per thread.
__global__ __launch_bounds__(256) void gla_bwd_gh_kernel(GlaBwdLaunch b, const unsigned* maxbits,
                                                         f16* gh) {
    const long long n8 = (long long)b.BH * b.L * kD / 8;
    const long long e = (long long)blockIdx.x * 256 + threadIdx.x;
    if (e >= n8) return;
    const float f = sigma_of(maxbits[0]) * b.scale;
    f16x8 o;
    if (b.do_f32) {
        const f32x4* s = reinterpret_cast<const f32x4*>(b.dout) + 2 * e;
        const f32x4 x0 = s[0], x1 = s[1];
#pragma unroll
        for (int i = 0; i < 4; ++i) { o[i] = (f16)(f * x0[i]); o[4 + i] = (f16)(f * x1[i]); }
    } else {
        const bf16x8 x = reinterpret_cast<const bf16x8*>(b.dout)[e];
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i] = (f16)(f * bf2f(x[i]));
    }
    reinterpret_cast<f16x8*>(gh)[e] = o;
}

// Enqueue chunk c's operand block and its 64-column tile of gh into an LDS stage
// (the layout of the forward scan's stage, gh in place of V).
__device__ __forceinline__ void issue_rchunk(char* stage, const char* blocks, const f16* gh,
                                             long long L, int bh, int tile, long long c,
                                             long long nch, int wave, int lane) {
    const char* blk = blocks + (size_t)((long long)bh * nch + c) * kChunkBytes;
#pragma unroll
    for (int i = 0; i < 12; ++i) {
        const int q = 12 * wave + i;
        dma16p(blk + 1024 * q + 16 * lane, stage + 1024 * q);
    }
    if (wave == 0 && lane < kTailChunks) dma16p(blk + kBlockMain + 16 * lane, stage + kBlockMain);
    const long long t0 = c * kC;
    const int n = (int)min((long long)kC, L - t0);
    const f16* gb = gh + ((long long)bh * L + t0) * kD + tile * 64;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int p = 64 * (2 * wave + i) + lane;
        const int tok = p >> 3;
        const int cc = (p & 7) ^ swzv(tok);
        dma16p(gb + (long long)min(tok, n - 1) * kD + 8 * cc, stage + kOffV + 1024 * (2 * wave + i));
    }
}

// Reverse scan: dM (128 x 64 value columns of one (b, h)) in fp32 registers,
// laid out as the forward scan's state: lane (G, m) of wave w holds
// dM[16 kb + 4G + i][64 tile + 16 w + m].
__global__ __launch_bounds__(256) void gla_rscan_kernel(GlaBwdLaunch b, BwdWs w) {
    extern __shared__ __attribute__((aligned(1024))) char smem[];
    const int BH = b.BH;
    const int blk = blockIdx.x;
    int bh, tile;
    if ((BH & 7) == 0) { bh = (blk & 7) + 8 * (blk >> 4); tile = (blk >> 3) & 1; }
    else { bh = blk >> 1; tile = blk & 1; }
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int m = lane & 15, G = lane >> 4;
    const int colw = wave * 16 + m;
    const int col = tile * 64 + colw;
    const long long nch = (b.L + kC - 1) / kC;
    const float sig = sigma_of(w.maxbits[0]);

    float* st = b.dstate + (long long)bh * kD * kD;
    f32x4 dM[8];
#pragma unroll
    for (int kb = 0; kb < 8; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) dM[kb][i] = sig * st[(16 * kb + 4 * G + i) * kD + col];

    issue_rchunk(smem, w.blocks, w.gh, b.L, bh, tile, nch - 1, nch, wave, lane);
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
    for (long long cc = 0; cc < nch; ++cc) {
        const long long c = nch - 1 - cc;
        wait_vmcnt<0>();
        __syncthreads();
        if (c > 0) issue_rchunk(smem + ((cc + 1) & 1) * kStageBytes, w.blocks, w.gh, b.L, bh, tile,
                                c - 1, nch, wave, lane);
        const char* S = smem + (cc & 1) * kStageBytes;
        const float* esm = reinterpret_cast<const float*>(S + kOffE);
        const float* dsm = reinterpret_cast<const float*>(S + kOffD);
        const float* bsm = reinterpret_cast<const float*>(S + kOffB);
        const float* xsm = reinterpret_cast<const float*>(S + kOffX);
        {   // dL/dM_C of this chunk, for the gradient kernel
            f16* sd = w.dme + ((long long)bh * nch + c) * kD * kD + col;
#pragma unroll
            for (int kb = 0; kb < 8; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i) sd[(16 * kb + 4 * G + i) * kD] = (f16)dM[kb][i];
        }
        // K dM
        f16x8 bM[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) bM[ks] = bfrag(dM[2 * ks], dM[2 * ks + 1]);
        f32x4 KM[4];
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
            KM[rb] = zero4;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                KM[rb] = mfma16h(afragK(S + kOffK, 16 * rb + m, ks, G), bM[ks], KM[rb]);
        }
        f32x4 e4[4], d4[4], b4[4], x4[4];
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
            e4[rb] = *reinterpret_cast<const f32x4*>(esm + 16 * rb + 4 * G);
            x4[rb] = *reinterpret_cast<const f32x4*>(xsm + 16 * rb + 4 * G);
            d4[rb] = *reinterpret_cast<const f32x4*>(dsm + 16 * rb + 4 * G);
            b4[rb] = *reinterpret_cast<const f32x4*>(bsm + 16 * rb + 4 * G);
        }
        // Gb[16 rb + 4G + i][colw] by one transposed read per row block
        f16x4 g4[4];
        {
            typedef short s16x4 __attribute__((ext_vector_type(4)));
            typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
            const int j = m >> 2, a = m & 3;
            const int vc = 16 * wave + 4 * a;
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) {
                const int t = 16 * rb + 4 * G + j;
                const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(
                    S + kOffV + t * 128 + 16 * ((vc >> 3) ^ swzv(t)) + 2 * (vc & 7)));
                g4[rb] = __builtin_bit_cast(f16x4, r);
            }
        }
        const f16x8 gb[2] = {cat(g4[0], g4[1]), cat(g4[2], g4[3])};
        // dU = Pm^T Gb + diag(Dn) K dM   (Pm^T upper triangular)
        f32x4 dU[4];
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
            dU[rb] = mfma16h(afragTt(S + kOffP, rb, 1, lane), gb[1], zero4);
            if (rb < 2) dU[rb] = mfma16h(afragTt(S + kOffP, rb, 0, lane), gb[0], dU[rb]);
#pragma unroll
            for (int i = 0; i < 4; ++i) dU[rb][i] += d4[rb][i] * KM[rb][i];
        }
        // dR = T^T dU   (T^T upper triangular)
        const f16x8 ub[2] = {bfrag(dU[0], dU[1]), bfrag(dU[2], dU[3])};
        f32x4 dR[4];
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
            dR[rb] = mfma16h(afragTt(S + kOffT, rb, 1, lane), ub[1], zero4);
            if (rb < 2) dR[rb] = mfma16h(afragTt(S + kOffT, rb, 0, lane), ub[0], dR[rb]);
        }
        {
            f16* sr = w.dr + ((long long)bh * nch + c) * kC * kD + col;
#pragma unroll
            for (int rb = 0; rb < 4; ++rb)
#pragma unroll
                for (int i = 0; i < 4; ++i) sr[(16 * rb + 4 * G + i) * kD] = (f16)dR[rb][i];
        }
        // dM <- E_C dM + Q^T diag(E) Gb - K^T diag(beta Ep) dR
        f32x4 eg[4], nr[4];
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                eg[rb][i] = e4[rb][i] * (float)g4[rb][i];
                nr[rb][i] = -b4[rb][i] * x4[rb][i] * dR[rb][i];
            }
        const f16x8 egb[2] = {bfrag(eg[0], eg[1]), bfrag(eg[2], eg[3])};
        const f16x8 nrb[2] = {bfrag(nr[0], nr[1]), bfrag(nr[2], nr[3])};
        const float egC = esm[kC - 1];
#pragma unroll
        for (int kb = 0; kb < 8; ++kb) {
#pragma unroll
            for (int i = 0; i < 4; ++i) dM[kb][i] *= egC;
            dM[kb] = mfma16h(afragKt(S + kOffQ, kb, 0, lane), egb[0], dM[kb]);
            dM[kb] = mfma16h(afragKt(S + kOffQ, kb, 1, lane), egb[1], dM[kb]);
            dM[kb] = mfma16h(afragKt(S + kOffK, kb, 0, lane), nrb[0], dM[kb]);
            dM[kb] = mfma16h(afragKt(S + kOffK, kb, 1, lane), nrb[1], dM[kb]);
        }
    }
    const float inv = 1.f / sig;
#pragma unroll
    for (int kb = 0; kb < 8; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) st[(16 * kb + 4 * G + i) * kD + col] = dM[kb][i] * inv;
}

// ---------------------------------------------------------------------------------
// Chunk gradient kernel: one workgroup of 8 waves (two per SIMD, so that one
// wave's latencies overlap the other's) per chunk. Operands sit in LDS as
// row-major fp16 with padded rows; every product is C = A Bt^T with both
// operands contiguous along the contraction, on v_mfma_f32_16x16x32_f16.
// Output tile (mt, nt) of 16x16: lane (G, m) holds rows 16 mt + 4G + i, column
// 16 nt + m. [64 x 128] outputs: wave w owns columns 16w .. 16w + 15 (tile
// nt = w), all four row tiles. [64 x 64] outputs: wave w owns column tile
// nt = w & 3 and row tiles 2 (w >> 2), 2 (w >> 2) + 1.
constexpr int kGradThreads = 512;

constexpr int kLd = kD + 8;   // padded row (halfs) of a 128-wide operand
constexpr int kLc = kC + 8;   // padded row of a 64-wide operand

template <int K>
__device__ __forceinline__ void mm_wide(const f16* A, int lda, const f16* Bt, int ldb,
                                        f32x4 (&acc)[4], int wave, int lane) {
    const int m = lane & 15, G = lane >> 4;
#pragma unroll
    for (int k0 = 0; k0 < K; k0 += 32) {
        const f16x8 bf = *reinterpret_cast<const f16x8*>(Bt + (16 * wave + m) * ldb + k0 + 8 * G);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            const f16x8 af = *reinterpret_cast<const f16x8*>(A + (16 * mt + m) * lda + k0 + 8 * G);
            acc[mt] = mfma16h(af, bf, acc[mt]);
        }
    }
}

template <int K>
__device__ __forceinline__ void mm_cc(const f16* A, int lda, const f16* Bt, int ldb,
                                      f32x4 (&acc)[2], int wave, int lane) {
    const int m = lane & 15, G = lane >> 4;
#pragma unroll
    for (int k0 = 0; k0 < K; k0 += 32) {
        const f16x8 bf = *reinterpret_cast<const f16x8*>(Bt + (16 * (wave & 3) + m) * ldb + k0 + 8 * G);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int mt = 2 * (wave >> 2) + h;
            const f16x8 af = *reinterpret_cast<const f16x8*>(A + (16 * mt + m) * lda + k0 + 8 * G);
            acc[h] = mfma16h(af, bf, acc[h]);
        }
    }
}

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over the 16 lanes of a lane group (the 16 columns of a tile row), in
// registers: xor 1 and xor 2 inside each quad, then rotations by 4 and by 8
// inside the 16-lane row (DPP). Every lane of the group ends with the sum (the
// additions are associated differently per lane; callers read one lane). All 64
// lanes must be active.
__device__ __forceinline__ float group16_sum(float v) {
    v += dpp_mov<0xB1>(v);    // quad_perm [1, 0, 3, 2]
    v += dpp_mov<0x4E>(v);    // quad_perm [2, 3, 0, 1]
    v += dpp_mov<0x124>(v);   // row_ror:4
    v += dpp_mov<0x128>(v);   // row_ror:8
    return v;
}

__global__ __launch_bounds__(kGradThreads) void gla_grad_kernel(GlaBwdLaunch b, BwdWs w) {
    __shared__ __attribute__((aligned(16))) f16 Kr[kC * kLd];     // K   [64][128]
    __shared__ __attribute__((aligned(16))) f16 KT[kD * kLc];     // K^T [128][64]
    __shared__ __attribute__((aligned(16))) f16 QT[kD * kLc];     // Q^T [128][64]
    __shared__ __attribute__((aligned(16))) f16 Gr[kC * kLd];     // Gb  [64][128]
    __shared__ __attribute__((aligned(16))) f16 Rr[kC * kLd];     // dR  [64][128]
    __shared__ __attribute__((aligned(16))) f16 Ur[kC * kLd];     // U   [64][128]
    __shared__ __attribute__((aligned(16))) f16 Mb[kD * kLd];     // M0, then dM_C; then 3 [64][64]
    __shared__ float gs[kC], gps[kC], Es[kC], Dn[kC], bs[kC], Eps[kC], als[kC];
    // per-wave partial row sums of dL/dg, dL/dgp and dL/dbeta: each wave adds
    // only to its own slice (one lane per row per instruction), and the slices
    // are summed in wave order at the end, so the result does not depend on
    // timing (no float atomics)
    __shared__ float pdg[kGradThreads / 64][kC], pdgp[kGradThreads / 64][kC], pdbt[kGradThreads / 64][kC];
    __shared__ float red[kGradThreads / 64];

    const long long nch = (b.L + kC - 1) / kC;
    const int cid = blockIdx.x;
    const int bh = cid / (int)nch;
    const long long c = cid - (long long)bh * nch;
    const long long t0 = c * kC;
    const int n = (int)min((long long)kC, b.L - t0);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int m = lane & 15, G = lane >> 4;
    const float sig = sigma_of(w.maxbits[0]);
    const float svv = sigma_of(w.maxbits[1]);          // the forward ran on sigma_v (v, M_0)
    const long long tok0 = (long long)bh * b.L + t0;   // first token row of the chunk
    const long long ci = (long long)bh * nch + c;      // chunk index
    // Pm at this lane's phase-4 positions (rows 16 mt + 4G + i of the wave's two row
    // tiles, column 16 (wave & 3) + m), fetched with the other operands rather than
    // inside phase 4
    const char* pmb = w.blocks + (size_t)ci * kChunkBytes + kOffP;
    f16 pmv[8];
#pragma unroll
    for (int r = 0; r < 8; ++r)
        pmv[r] = *reinterpret_cast<const f16*>(
            pmb + offT(16 * (2 * (wave >> 2) + (r >> 2)) + 4 * G + (r & 3), 16 * (wave & 3) + m));

    // ---- phase 0: stage operands (rows >= n zero) and per-token factors. Every
    // global operand of the chunk is requested first, so that the loads are in
    // flight together; dM_C and V stay in registers until they are used.
    const f16* m0g = w.save_m + ci * kD * kD;
    const f16* dmg = w.dme + ci * kD * kD;
    bf16x8 kin[2], qin[2], vin[2];
    f16x8 gin[2], rin[2], uin[2], m0in[4], dmin[4];
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        const int e = tid + kGradThreads * it, row = e >> 4, c8 = (e & 15) * 8;
        if (row < n) {
            const long long tr = (tok0 + row) * kD + c8, cr = (ci * kC + row) * kD + c8;
            kin[it] = *reinterpret_cast<const bf16x8*>(static_cast<const bf16*>(b.k) + tr);
            qin[it] = *reinterpret_cast<const bf16x8*>(static_cast<const bf16*>(b.q) + tr);
            vin[it] = *reinterpret_cast<const bf16x8*>(static_cast<const bf16*>(b.v) + tr);
            gin[it] = *reinterpret_cast<const f16x8*>(w.gh + tr);
            rin[it] = *reinterpret_cast<const f16x8*>(w.dr + cr);
            uin[it] = *reinterpret_cast<const f16x8*>(w.save_u + cr);
        }
    }
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        const int e = tid + kGradThreads * it, row = e >> 4, c8 = (e & 15) * 8;
        m0in[it] = *reinterpret_cast<const f16x8*>(m0g + row * kD + c8);
        dmin[it] = *reinterpret_cast<const f16x8*>(dmg + row * kD + c8);
    }
    if (wave == 0) {
        float la = 0.f, a = 1.f;
        if (lane < n) {
            a = b.alpha[tok0 + lane];
            const float lg = logf(a);
            la = (lg < kLogFloor) ? kLogFloor : lg;
        }
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float y = __shfl_up(la, off, 64);
            if (lane >= off) la += y;
        }
        const float gC = __shfl(la, 63, 64);
        const float prev = __shfl_up(la, 1, 64);
        const float gp = b.form ? (lane == 0 ? 0.f : prev) : la;
        gs[lane] = la;
        gps[lane] = gp;
        Es[lane] = __expf(la);
        Dn[lane] = __expf(gC - la);
        Eps[lane] = __expf(gp);
        bs[lane] = lane < n ? b.beta[tok0 + lane] : 0.f;
        als[lane] = a;
    }
    pdg[wave][lane] = 0.f;
    pdgp[wave][lane] = 0.f;
    pdbt[wave][lane] = 0.f;
    // (the chunk's global operands were all requested at the top: see phase 0)
#pragma unroll
    for (int it = 0; it < 2; ++it) {   // 16-byte pieces of 64 rows x 128
        const int e = tid + kGradThreads * it, row = e >> 4, c8 = (e & 15) * 8;
        f16x8 kk, qq, gg, rr, uu;
        if (row < n) {
#pragma unroll
            for (int i = 0; i < 8; ++i) { kk[i] = (f16)bf2f(kin[it][i]); qq[i] = (f16)bf2f(qin[it][i]); }
            gg = gin[it];
            rr = rin[it];
            uu = uin[it];
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) { kk[i] = 0; qq[i] = 0; gg[i] = 0; rr[i] = 0; uu[i] = 0; }
        }
        *reinterpret_cast<f16x8*>(Kr + row * kLd + c8) = kk;
        *reinterpret_cast<f16x8*>(Gr + row * kLd + c8) = gg;
        *reinterpret_cast<f16x8*>(Rr + row * kLd + c8) = rr;
        *reinterpret_cast<f16x8*>(Ur + row * kLd + c8) = uu;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            KT[(c8 + i) * kLc + row] = kk[i];
            QT[(c8 + i) * kLc + row] = qq[i];
        }
    }
    float sdot = 0.f;   // <dM_C, M0>
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        const int e = tid + kGradThreads * it, row = e >> 4, c8 = (e & 15) * 8;
        *reinterpret_cast<f16x8*>(Mb + row * kLd + c8) = m0in[it];
#pragma unroll
        for (int i = 0; i < 8; ++i) sdot += (float)m0in[it][i] * (float)dmin[it][i];
    }
    sdot = wave_sum(sdot);
    if (lane == 0) red[wave] = sdot;
    __syncthreads();
    if (tid == 0) {
        float t = 0.f;
#pragma unroll
        for (int i = 0; i < kGradThreads / 64; ++i) t += red[i];
        pdg[0][kC - 1] += Es[kC - 1] * t;
    }

    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
    f32x4 accQ[4], accK[4], X[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) { accQ[t] = zero4; accK[t] = zero4; }

    // ---- phase 1: Gb M0^T -> dQ (diag(E)), dg += E_i Q_i . (Gb M0^T)_i
#pragma unroll
    for (int t = 0; t < 4; ++t) X[t] = zero4;
    mm_wide<kD>(Gr, kLd, Mb, kLd, X, wave, lane);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 16 * mt + 4 * G + i;
            const int col = 16 * wave + m;
            accQ[mt][i] = Es[row] * X[mt][i];
            float s = (float)QT[col * kLc + row] * X[mt][i];
            s = group16_sum(s);
            if (m == 0) pdg[wave][row] += Es[row] * s;
        }
    // ---- phase 2: dR M0^T -> dK (-diag(beta Ep)); dgp, dbeta
#pragma unroll
    for (int t = 0; t < 4; ++t) X[t] = zero4;
    mm_wide<kD>(Rr, kLd, Mb, kLd, X, wave, lane);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 16 * mt + 4 * G + i;
            const int col = 16 * wave + m;
            accK[mt][i] = -bs[row] * Eps[row] * X[mt][i];
            float s = (float)Kr[row * kLd + col] * X[mt][i];
            s = group16_sum(s);
            if (m == 0) {
                pdgp[wave][row] += -bs[row] * Eps[row] * s;
                pdbt[wave][row] += -Eps[row] * s;
            }
        }
    __syncthreads();   // every wave is done with M0
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        const int e = tid + kGradThreads * it, row = e >> 4, c8 = (e & 15) * 8;
        *reinterpret_cast<f16x8*>(Mb + row * kLd + c8) = dmin[it];
    }
    __syncthreads();
    // ---- phase 3: U dM_C^T -> dK (diag(Dn)); dg terms of M_C
#pragma unroll
    for (int t = 0; t < 4; ++t) X[t] = zero4;
    mm_wide<kD>(Ur, kLd, Mb, kLd, X, wave, lane);
    float slast = 0.f;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 16 * mt + 4 * G + i;
            const int col = 16 * wave + m;
            accK[mt][i] += Dn[row] * X[mt][i];
            float s = (float)Kr[row * kLd + col] * X[mt][i];
            s = group16_sum(s) * Dn[row];
            if (m == 0) {
                pdg[wave][row] -= s;
                slast += s;
            }
        }
    slast += __shfl_xor(slast, 16, 64);   // the four m == 0 lanes, summed in one lane
    slast += __shfl_xor(slast, 32, 64);
    if (lane == 0) pdg[wave][kC - 1] += slast;
    __syncthreads();   // Mb free: three 64 x 64 buffers
    f16* D1 = Mb;
    f16* D1T = Mb + kC * kLc;
    f16* Bs = Mb + 2 * kC * kLc;
    // ---- phase 4: Gb U^T -> D1 = (.) o Gamma (incl. lower), dg from Pm
    {
        f32x4 C4[2] = {zero4, zero4};
        mm_cc<kD>(Gr, kLd, Ur, kLd, C4, wave, lane);
        const int j = 16 * (wave & 3) + m;
        float colsum = 0.f;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 16 * (2 * (wave >> 2) + h) + 4 * G + i;
                const float x = C4[h][i];
                const float pm = (float)pmv[4 * h + i];
                const float y = x * pm;
                const float rs = group16_sum(y);
                if (m == 0) pdg[wave][row] += rs;
                colsum += y;
                const float d1 = j <= row ? x * __expf(gs[row] - gs[j]) : 0.f;
                D1[row * kLc + j] = (f16)d1;
                D1T[j * kLc + row] = (f16)d1;
            }
        colsum += __shfl_xor(colsum, 16, 64);
        colsum += __shfl_xor(colsum, 32, 64);
        if (G == 0) pdg[wave][j] -= colsum;
    }
    // ---- phase 5: dA = -strictly-lower(dR U^T), K K^T -> dbeta, dgp, dg, Bs
    {
        f32x4 P5[2] = {zero4, zero4}, KK[2] = {zero4, zero4};
        mm_cc<kD>(Rr, kLd, Ur, kLd, P5, wave, lane);
        mm_cc<kD>(Kr, kLd, Kr, kLd, KK, wave, lane);
        const int j = 16 * (wave & 3) + m;
        float colsum = 0.f;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 16 * (2 * (wave >> 2) + h) + 4 * G + i;
                float bm = 0.f, zk = 0.f, da_a = 0.f;
                if (j < row) {
                    const float lam = __expf(gps[row] - gs[j]);
                    const float dA = -P5[h][i];
                    const float z = dA * lam;
                    zk = z * KK[h][i];
                    da_a = dA * bs[row] * KK[h][i] * lam;
                    bm = bs[row] * z;
                }
                const float r1 = group16_sum(zk), r2 = group16_sum(da_a);
                if (m == 0) { pdbt[wave][row] += r1; pdgp[wave][row] += r2; }
                colsum += da_a;
                if (j < row) { Bs[row * kLc + j] = (f16)bm; Bs[j * kLc + row] = (f16)bm; }
                else if (j == row) Bs[row * kLc + j] = (f16)0.f;
            }
        colsum += __shfl_xor(colsum, 16, 64);
        colsum += __shfl_xor(colsum, 32, 64);
        if (G == 0) pdg[wave][j] -= colsum;
    }
    __syncthreads();
    // ---- phase 6: dQ += D1 K, dK += D1^T Q + Bs K
    mm_wide<kC>(D1, kLc, KT, kLc, accQ, wave, lane);
    mm_wide<kC>(D1T, kLc, QT, kLc, accK, wave, lane);
    mm_wide<kC>(Bs, kLc, KT, kLc, accK, wave, lane);
    // ---- phase 7: outputs (scaled back by 1/sigma; those that scale with the
    // forward's values, dq, dk, dalpha, dbeta, also by 1/sigma_v)
    const float inv = 1.f / sig, invv = inv / svv;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 16 * mt + 4 * G + i;
            if (row < n) {
                const long long o = (tok0 + row) * kD + 16 * wave + m;
                const float xq = accQ[mt][i] * invv, xk = accK[mt][i] * invv;
                if (b.grad_f32) {
                    static_cast<float*>(b.dq)[o] = xq;
                    static_cast<float*>(b.dk)[o] = xk;
                } else {
                    static_cast<bf16*>(b.dq)[o] = f2bf(xq);
                    static_cast<bf16*>(b.dk)[o] = f2bf(xk);
                }
            }
        }
    // dV = diag(beta) dR; dbeta += dR_i . V_i (16 lanes per row)
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        const int e = tid + kGradThreads * it, row = e >> 4, c8 = (e & 15) * 8;
        float s = 0.f;
        if (row < n) {
            const bf16x8 vv = vin[it];
            float ov[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float r = (float)Rr[row * kLd + c8 + i];
                s += r * (bf2f(vv[i]) * svv);
                ov[i] = bs[row] * r * inv;
            }
            const long long o = (tok0 + row) * kD + c8;
            if (b.grad_f32) {
                f32x4* d = reinterpret_cast<f32x4*>(static_cast<float*>(b.dv) + o);
                d[0] = f32x4{ov[0], ov[1], ov[2], ov[3]};
                d[1] = f32x4{ov[4], ov[5], ov[6], ov[7]};
            } else {
                bf16x8 ob;
#pragma unroll
                for (int i = 0; i < 8; ++i) ob[i] = f2bf(ov[i]);
                *reinterpret_cast<bf16x8*>(static_cast<bf16*>(b.dv) + o) = ob;
            }
        }
        s = group16_sum(s);
        if ((e & 15) == 0 && row < n) pdbt[wave][row] += s;
    }
    __syncthreads();
    if (wave == 0) {
        // dlog(alpha)_r = sum_{i >= r} dg_i + sum_{i >= r} dgp_i (form 0) or sum_{i > r} dgp_i
        float x = 0.f, y = 0.f, zb = 0.f;
#pragma unroll
        for (int v8 = 0; v8 < kGradThreads / 64; ++v8) {
            x += pdg[v8][lane];
            y += pdgp[v8][lane];
            zb += pdbt[v8][lane];
        }
        float sx = x, sy = y;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float ax = __shfl_down(sx, off, 64), ay = __shfl_down(sy, off, 64);
            if (lane + off < 64) { sx += ax; sy += ay; }
        }
        const float dla = sx + (b.form ? sy - y : sy);
        if (lane < n) {
            b.dalpha[tok0 + lane] = dla / als[lane] * invv;
            b.dbeta[tok0 + lane] = zb * invv;
        }
    }
}

}  // namespace

size_t gla_bwd_workspace_bytes(int dtype, int BH, long long L, int d) {
    const long long nck = (L + kCk - 1) / kCk;
    if (dtype == 0)
        return (size_t)BH * (size_t)((nck + 1) + (kCk + 1)) * (size_t)d * d * sizeof(float);
    return bwd_ws_bytes(BH, L);
}

hipError_t launch_gla_bwd(const GlaBwdLaunch& b, hipStream_t stream) {
    if (b.BH == 0 || b.L == 0) return hipSuccess;
    if (b.ws_bytes < gla_bwd_workspace_bytes(b.dtype, b.BH, b.L, b.d)) return hipErrorInvalidValue;
    if (b.dtype == 0) {
        if (b.d == 64)
            hipLaunchKernelGGL((gla_bwd_f32_kernel<64>), dim3(b.BH), dim3(256), 0, stream, b);
        else
            hipLaunchKernelGGL((gla_bwd_f32_kernel<128>), dim3(b.BH), dim3(256), 0, stream, b);
        return hipGetLastError();
    }
    if (b.d != kD || b.chunk != kC) return hipErrorInvalidValue;
    // bf16: forward prep + scan (saving M0, U), sigma, gh, reverse scan, gradients
    const long long nch = (b.L + kC - 1) / kC;
    if ((long long)b.BH * nch > 0x7fffffffLL) return hipErrorInvalidValue;
    BwdWs w = bwd_ws(b.ws, b.BH, b.L);
    hipError_t e;
    if ((e = launch_fill_f32(w.state, b.state0, (long long)b.BH * kD * kD, stream)) != hipSuccess) return e;
    if ((e = launch_fill_f32(reinterpret_cast<float*>(w.maxbits), nullptr, 2, stream)) != hipSuccess) return e;
    const long long nd = (long long)b.BH * b.L * kD;
    const long long gmax = min(1024LL, (nd + 255) / 256);
    hipLaunchKernelGGL(gla_bwd_max_kernel, dim3((unsigned)gmax), dim3(256), 0, stream, b, w.maxbits);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    GlaLaunch g;
    memset(&g, 0, sizeof(g));
    g.q = b.q; g.k = b.k; g.v = b.v; g.alpha = b.alpha; g.beta = b.beta;
    g.state = w.state; g.o = nullptr; g.out_f32 = 1;
    g.L = b.L; g.BH = b.BH; g.d = b.d; g.chunk = b.chunk; g.scale = b.scale; g.dtype = b.dtype;
    g.form = b.form;
    g.ws = w.blocks;
    g.ws_bytes = (size_t)b.BH * nch * kChunkBytes;
    g.save_m = w.save_m;
    g.save_u = w.save_u;
    g.vscale = w.maxbits + 1;
    if ((e = launch_gla_bf16(g, stream)) != hipSuccess) return e;
    const long long n8 = (nd / 8 + 255) / 256;
    hipLaunchKernelGGL(gla_bwd_gh_kernel, dim3((unsigned)n8), dim3(256), 0, stream, b,
                       (const unsigned*)w.maxbits, w.gh);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const size_t smem = 2 * kStageBytes;
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(gla_rscan_kernel),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(gla_rscan_kernel, dim3((unsigned)(b.BH * 2)), dim3(256), smem, stream, b, w);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(gla_grad_kernel, dim3((unsigned)(b.BH * nch)), dim3(kGradThreads), 0, stream, b, w);
    return hipGetLastError();
}

}  // namespace hta
