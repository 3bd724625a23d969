// gla_f32.hip -- chunked gated-delta GLA, fp32 end to end (vector ALU).
//
// Method: page "Kairos：面向物理 AI 的原生世界模型栈" (yingwang.github.io), section
// 二、方法, GLA paragraph and update equations (GatedDeltaNet reading):
//   S_t = alpha_t (S_{t-1} - beta_t (S_{t-1} k_t) k_t^T) + beta_t v_t k_t^T,  o_t = S_t q_t.
// The state is kept as M = S^T (dk x dv). Over a chunk of n tokens from M0,
// with g = inclusive cumulative sum of log alpha inside the chunk:
//   (I + A) [W | U~] = [diag(beta e^g) K | diag(beta) V],
//        A = strictly-lower( diag(beta) (K K^T o e^{g_i - g_j}) )
//   U   = U~ - W M0
//   O   = diag(e^g) Q M0 + tril(Q K^T o e^{g_i - g_j}) U
//   M_n = e^{g_n} M0 + K^T diag(e^{g_n - g}) U
// (unrolling u_t = beta_t (v_t - alpha_t S_{t-1} k_t) through the chunk).
//
// One workgroup per (batch, head) walks the chunks in order; the state and the
// chunk's W, U, A live in LDS. This path serves fp32 inputs (small workloads)
// and checks the chunk algebra at fp32 precision; the bf16 path is separate.
#include "device_common.h"
#include "hta_internal.h"

namespace hta {

namespace {

constexpr float kLogFloor = -1.0e4f;   // log(alpha) floor: alpha = 0 decays to exactly 0

template <int D, int C>
__global__ __launch_bounds__(256) void gla_f32_kernel(GlaLaunch g) {
    __shared__ float Ms[D * D];        // M[r][c]
    __shared__ float Ws[C * D];        // W[i][r]
    __shared__ float Us[C * D];        // U~ then U: [i][c]
    __shared__ float As[C * C];        // A, then Pm
    __shared__ float gs[C];
    __shared__ float egs[C];
    __shared__ float gps[C];    // decay exponent of the erase path: g_i, or g_{i-1} (printed form)
    __shared__ float egps[C];

    const int bh = blockIdx.x;
    const int tid = threadIdx.x;
    const long long L = g.L;
    const float* q = static_cast<const float*>(g.q) + (long long)bh * L * D;
    const float* k = static_cast<const float*>(g.k) + (long long)bh * L * D;
    const float* v = static_cast<const float*>(g.v) + (long long)bh * L * D;
    const float* al = g.alpha + (long long)bh * L;
    const float* be = g.beta + (long long)bh * L;
    float* st = g.state + (long long)bh * D * D;
    float* o = g.o ? static_cast<float*>(g.o) + (long long)bh * L * D : nullptr;

    for (int e = tid; e < D * D; e += 256) Ms[e] = st[e];
    __syncthreads();

    for (long long t0 = 0; t0 < L; t0 += C) {
        const int n = (int)((L - t0) < C ? (L - t0) : C);
        const float* Kc = k + t0 * D;
        const float* Vc = v + t0 * D;
        const float* Qc = q + t0 * D;
        if (tid == 0) {
            float acc = 0.f;
            for (int i = 0; i < n; ++i) {
                const float lg = logf(al[t0 + i]);
                const float prev = acc;
                acc += (lg < kLogFloor) ? kLogFloor : lg;   // NaN passes through
                gs[i] = acc;
                egs[i] = expf(acc);
                gps[i] = g.form ? prev : acc;
                egps[i] = expf(gps[i]);
            }
        }
        __syncthreads();
        // A[i][j] = beta_i e^{gp_i - g_j} k_i.k_j for j < i (gp = g, or g_{i-1} for the
        // printed form, whose erase term reads the state before the decay).
        for (int e = tid; e < n * n; e += 256) {
            const int i = e / n, j = e - i * n;
            float a = 0.f;
            if (j < i) {
                float s = 0.f;
                for (int r = 0; r < D; ++r) s += Kc[i * D + r] * Kc[j * D + r];
                a = be[t0 + i] * expf(gps[i] - gs[j]) * s;
            }
            As[i * C + j] = a;
        }
        __syncthreads();
        // Forward substitution, one right-hand-side column per thread.
        for (int col = tid; col < 2 * D; col += 256) {
            const bool isW = col < D;
            const int cc = isW ? col : col - D;
            float* X = isW ? Ws : Us;
            for (int i = 0; i < n; ++i) {
                float x = isW ? be[t0 + i] * egps[i] * Kc[i * D + cc] : be[t0 + i] * Vc[i * D + cc];
                for (int j = 0; j < i; ++j) x -= As[i * C + j] * X[j * D + cc];
                X[i * D + cc] = x;
            }
        }
        __syncthreads();
        // U = U~ - W M0 ; Pm = tril(Q K^T o Gamma) (A no longer needed).
        for (int e = tid; e < n * D; e += 256) {
            const int i = e / D, c = e - i * D;
            float s = 0.f;
            for (int r = 0; r < D; ++r) s += Ws[i * D + r] * Ms[r * D + c];
            Us[i * D + c] -= s;
        }
        for (int e = tid; e < n * n; e += 256) {
            const int i = e / n, j = e - i * n;
            float pm = 0.f;
            if (j <= i) {
                float s = 0.f;
                for (int r = 0; r < D; ++r) s += Qc[i * D + r] * Kc[j * D + r];
                pm = expf(gs[i] - gs[j]) * s;
            }
            As[i * C + j] = pm;
        }
        __syncthreads();
        // O = diag(e^g) Q M0 + Pm U.
        if (o) {
            for (int e = tid; e < n * D; e += 256) {
                const int i = e / D, c = e - i * D;
                float s = 0.f;
                for (int r = 0; r < D; ++r) s += Qc[i * D + r] * Ms[r * D + c];
                float u = 0.f;
                for (int j = 0; j <= i; ++j) u += As[i * C + j] * Us[j * D + c];
                o[(t0 + i) * D + c] = g.scale * (egs[i] * s + u);
            }
        }
        __syncthreads();
        // M = e^{g_n} M0 + K^T diag(e^{g_n - g}) U.
        const float gl = gs[n - 1];
        for (int e = tid; e < D * D; e += 256) {
            const int r = e / D, c = e - r * D;
            float s = 0.f;
            for (int i = 0; i < n; ++i) s += expf(gl - gs[i]) * Kc[i * D + r] * Us[i * D + c];
            Ms[e] = egs[n - 1] * Ms[e] + s;
        }
        __syncthreads();
    }
    for (int e = tid; e < D * D; e += 256) st[e] = Ms[e];
}

template <int D>
hipError_t launch_f32_d(const GlaLaunch& g, hipStream_t s) {
    const dim3 grid(g.BH), block(256);
    switch (g.chunk) {
        case 16: hipLaunchKernelGGL((gla_f32_kernel<D, 16>), grid, block, 0, s, g); break;
        case 32: hipLaunchKernelGGL((gla_f32_kernel<D, 32>), grid, block, 0, s, g); break;
        case 64: hipLaunchKernelGGL((gla_f32_kernel<D, 64>), grid, block, 0, s, g); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gla_f32(const GlaLaunch& g, hipStream_t stream) {
    if (g.BH == 0 || g.L == 0) return hipSuccess;
    return g.d == 64 ? launch_f32_d<64>(g, stream) : launch_f32_d<128>(g, stream);
}

}  // namespace hta
