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
#include <type_traits>

#include "device_common.h"
#include "hta_internal.h"

namespace hta {

namespace {

constexpr int kCk = 64;                // tokens per checkpoint segment
constexpr float kLogFloor = -1.0e4f;   // log(alpha) floor of the chunked forms

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

}  // namespace

size_t gla_bwd_workspace_bytes(int dtype, int BH, long long L, int d) {
    const long long nck = (L + kCk - 1) / kCk;
    if (dtype == 0)
        return (size_t)BH * (size_t)((nck + 1) + (kCk + 1)) * (size_t)d * d * sizeof(float);
    return 0;
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
    return hipErrorInvalidValue;
}

}  // namespace hta
