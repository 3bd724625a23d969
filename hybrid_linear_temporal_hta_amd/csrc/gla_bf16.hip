// gla_bf16.hip -- chunked gated-delta GLA on bf16 MFMA (gfx950), fp32 state.
//
// Method: page "Kairos：面向物理 AI 的原生世界模型栈" (yingwang.github.io), section
// 二、方法, GLA paragraph and update equations, GatedDeltaNet reading:
//   S_t = alpha_t (S_{t-1} - beta_t (S_{t-1} k_t) k_t^T) + beta_t v_t k_t^T,  o_t = S_t q_t.
// State M = S^T (dk x dv). For a chunk of C = 64 tokens from M0 with g the
// inclusive cumulative sum of log alpha inside the chunk (the UT / WY form):
//   T = (I + A)^-1,  A = strictly-lower( diag(beta) (K K^T o e^{g_i - g_j}) )
//   U = T X,         X = diag(beta) (V - diag(e^g) (K M0))
//   O = diag(e^g) (Q M0) + Pm U,       Pm = tril(Q K^T o e^{g_i - g_j})
//   M = e^{g_C} M0 + K^T (diag(e^{g_C - g}) U)
//
// Precision: the inputs are bf16 and every accumulation is fp32; the operands
// the kernels build themselves (T, Pm, the state copy fed to K M0 / Q M0, X,
// U) are rounded to fp16, whose 11-bit significand keeps the chunk algebra
// about 8x closer to the exact result than bf16 operands would (bf16 inputs
// convert to fp16 exactly). fp16 bounds their range: |v| and |state| must stay
// below 65504 (with unit-norm keys, as the contraction of the update needs).
//
// Two kernels:
//   prep (one workgroup per chunk, all chunks in parallel): g, A and Pm from
//     K K^T and Q K^T on v_mfma_f32_32x32x16_bf16, then T by a register-resident
//     forward substitution in fp32 (4 lanes per column, 16 columns per wave).
//     Writes T and Pm (fp16) and g (fp32) per chunk to the workspace.
//   scan (one workgroup per (batch, head, 64 value columns), chunks in order):
//     each wave owns 16 value columns of the fp32 state as eight 16x16 MFMA
//     accumulator tiles. K M0, Q M0, T X, Pm U and K^T U run on
//     v_mfma_f32_16x16x32_f16; every product whose B operand is a previous
//     result (M0, X, U) takes it straight from the accumulator registers, the
//     token/key order inside a k-step being permuted identically in A and B,
//     so the state never leaves registers. K, K^T (transposed on the way in),
//     Q, T, Pm, g and beta of the next chunk are staged through LDS (double
//     buffered) while the current chunk computes.
#include "device_common.h"
#include "hta_internal.h"

namespace hta {

namespace {

constexpr int kC = 64;                 // chunk
constexpr int kD = 128;                // head dim
constexpr float kLogFloor = -1.0e4f;   // log(alpha) floor: alpha = 0 decays to exactly 0
constexpr size_t kChunkBytes = 2 * kC * kC * 2 + kC * 4;   // T, Pm (fp16) + g (fp32)

__device__ __forceinline__ char* chunk_ws(void* ws, long long cid) {
    return static_cast<char*>(ws) + (size_t)cid * kChunkBytes;
}

// ------------------------------------------------------------------ prep

constexpr int kKsP = kD + 8;      // padded K row (bf16)
constexpr int kAsP = 68;          // padded A row (fp32), permuted columns

__global__ __launch_bounds__(256) void gla_prep_bf16_kernel(GlaLaunch g, int nch) {
    __shared__ __attribute__((aligned(16))) bf16 Ks[kC * kKsP];
    __shared__ __attribute__((aligned(16))) float As[kC * kAsP];   // A[i][(j&3)*16 + (j>>2)]
    __shared__ float gs[kC];
    __shared__ float bs[kC];

    const int cid = blockIdx.x;
    const int bh = cid / nch, c = cid - bh * nch;
    const long long t0 = (long long)c * kC;
    const int n = (int)min((long long)kC, g.L - t0);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const bf16* kp = static_cast<const bf16*>(g.k) + ((long long)bh * g.L + t0) * kD;
    const bf16* qp = static_cast<const bf16*>(g.q) + ((long long)bh * g.L + t0) * kD;
    char* wsc = chunk_ws(g.ws, cid);
    f16* Tw = reinterpret_cast<f16*>(wsc);
    f16* Pw = Tw + kC * kC;
    float* gw = reinterpret_cast<float*>(Pw + kC * kC);

#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int ci = tid + 256 * r, row = ci >> 4, col = (ci & 15) * 8;
        u32x4 val = {0u, 0u, 0u, 0u};
        if (row < n) val = *reinterpret_cast<const u32x4*>(kp + (long long)row * kD + col);
        *reinterpret_cast<u32x4*>(Ks + row * kKsP + col) = val;
    }
    if (wave == 0) {
        // inclusive prefix sum of log(alpha) over the chunk (alpha = 1 past the end)
        float la = 0.f;
        if (lane < n) {
            const float lg = logf(g.alpha[(long long)bh * g.L + t0 + lane]);
            la = (lg < kLogFloor) ? kLogFloor : lg;   // NaN passes through
        }
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float y = __shfl_up(la, off, 64);
            if (lane >= off) la += y;
        }
        gs[lane] = la;
        gw[lane] = la;
        bs[lane] = lane < n ? g.beta[(long long)bh * g.L + t0 + lane] : 0.f;
    }
    __syncthreads();

    // K K^T and Q K^T, one 32x32 block per wave.
    {
        const int mb = wave >> 1, nb = wave & 1;
        const int nn = lane & 31, h = lane >> 5;
        f32x16 kk, qk;
#pragma unroll
        for (int i = 0; i < 16; ++i) { kk[i] = 0.f; qk[i] = 0.f; }
        if (mb >= nb) {
            const int qrow = mb * 32 + nn;
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) {
                const bf16x8 ka = *reinterpret_cast<const bf16x8*>(Ks + (mb * 32 + nn) * kKsP + 16 * ks + 8 * h);
                const bf16x8 kb = *reinterpret_cast<const bf16x8*>(Ks + (nb * 32 + nn) * kKsP + 16 * ks + 8 * h);
                bf16x8 qa;
                if (qrow < n) qa = *reinterpret_cast<const bf16x8*>(qp + (long long)qrow * kD + 16 * ks + 8 * h);
                else
#pragma unroll
                    for (int j = 0; j < 8; ++j) qa[j] = (bf16)0.f;
                kk = mfma32(ka, kb, kk);
                qk = mfma32(qa, kb, qk);
            }
        }
        const int j = nb * 32 + nn;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int i = mb * 32 + 8 * (e >> 2) + 4 * h + (e & 3);
            const float dec = (j <= i) ? __expf(gs[i] - gs[j]) : 0.f;
            As[i * kAsP + (j & 3) * 16 + (j >> 2)] = (j < i) ? bs[i] * dec * kk[e] : 0.f;
            Pw[i * kC + j] = (f16)((j <= i) ? dec * qk[e] : 0.f);
        }
    }
    __syncthreads();

    // T = (I + A)^-1 by forward substitution: lane (col, sub) keeps x_j for j = sub (mod 4).
    {
        const int col = wave * 16 + (lane >> 2), sub = lane & 3;
        float x[16];
#pragma unroll
        for (int m = 0; m < 16; ++m) x[m] = 0.f;
#pragma unroll
        for (int i = 0; i < kC; ++i) {
            float part = 0.f;
            const float* arow = As + i * kAsP + sub * 16;
#pragma unroll
            for (int m4 = 0; m4 < (i + 15) / 16; ++m4) {
                const f32x4 a4 = *reinterpret_cast<const f32x4*>(arow + 4 * m4);
#pragma unroll
                for (int u = 0; u < 4; ++u) part += a4[u] * x[4 * m4 + u];
            }
            part += __shfl_xor(part, 1, 64);
            part += __shfl_xor(part, 2, 64);
            const float xi = (i == col ? 1.f : 0.f) - part;
            if ((i & 3) == sub) x[i >> 2] = xi;
        }
#pragma unroll
        for (int m = 0; m < 16; ++m) Tw[(sub + 4 * m) * kC + col] = (f16)x[m];
    }
}

// ------------------------------------------------------------------ scan

constexpr int kQP = kD + 8;    // Ks / Qs row stride
constexpr int kTP = kC + 8;    // Kt / Ts / Ps row stride

struct ScanBuf {                 // fp16 operands of the scan's products
    f16 Ks[kC * kQP];
    f16 Qs[kC * kQP];
    f16 Kt[kD * kTP];
    f16 Ts[kC * kTP];
    f16 Ps[kC * kTP];
    float gs[kC];
    float egs[kC];
    float bs[kC];
};

struct StageRegs {
    u32x4 k[4];
    u32x4 q[4];
    u32x4 t[2];
    u32x4 p[2];
    f32x4 gb;
};

__device__ __forceinline__ void stage_load(StageRegs& r, const GlaLaunch& g, int bh, long long c,
                                           int tid) {
    const long long t0 = c * kC;
    const int n = (int)min((long long)kC, g.L - t0);
    const bf16* kp = static_cast<const bf16*>(g.k) + ((long long)bh * g.L + t0) * kD;
    const bf16* qp = static_cast<const bf16*>(g.q) + ((long long)bh * g.L + t0) * kD;
    const int kg = tid & 15, dg = tid >> 4;
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
        const int tok = 4 * kg + r4;
        r.k[r4] = tok < n ? *reinterpret_cast<const u32x4*>(kp + (long long)tok * kD + 8 * dg)
                          : u32x4{0u, 0u, 0u, 0u};
        const int ci = tid + 256 * r4, row = ci >> 4, col = (ci & 15) * 8;
        r.q[r4] = row < n ? *reinterpret_cast<const u32x4*>(qp + (long long)row * kD + col)
                          : u32x4{0u, 0u, 0u, 0u};
    }
    const f16* Tw = reinterpret_cast<const f16*>(chunk_ws(g.ws, (long long)bh * ((g.L + kC - 1) / kC) + c));
    const f16* Pw = Tw + kC * kC;
    const float* gw = reinterpret_cast<const float*>(Pw + kC * kC);
#pragma unroll
    for (int r2 = 0; r2 < 2; ++r2) {
        const int ci = tid + 256 * r2;
        r.t[r2] = *reinterpret_cast<const u32x4*>(Tw + ci * 8);
        r.p[r2] = *reinterpret_cast<const u32x4*>(Pw + ci * 8);
    }
    if (tid < 16) {
        r.gb = *reinterpret_cast<const f32x4*>(gw + 4 * tid);
    } else if (tid < 32) {
        const int b0 = 4 * (tid - 16);
        const float* bp = g.beta + (long long)bh * g.L + t0;
#pragma unroll
        for (int u = 0; u < 4; ++u) r.gb[u] = (b0 + u < n) ? bp[b0 + u] : 0.f;
    }
}

__device__ __forceinline__ void stage_store(const StageRegs& r, ScanBuf& b, int tid) {
    const int kg = tid & 15, dg = tid >> 4;
    u32x4 kh[4];                             // K as fp16 (exact)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
        kh[r4] = bf16x8_to_f16x8(r.k[r4]);
        *reinterpret_cast<u32x4*>(b.Ks + (4 * kg + r4) * kQP + 8 * dg) = kh[r4];
    }
#pragma unroll
    for (int w = 0; w < 4; ++w) {            // transpose 4 tokens x 8 dims into Kt[dim][token]
        const uint32_t a0 = kh[0][w], a1 = kh[1][w], a2 = kh[2][w], a3 = kh[3][w];
        u32x2 lo, hi;
        lo[0] = (a0 & 0xffffu) | (a1 << 16);
        lo[1] = (a2 & 0xffffu) | (a3 << 16);
        hi[0] = (a0 >> 16) | (a1 & 0xffff0000u);
        hi[1] = (a2 >> 16) | (a3 & 0xffff0000u);
        *reinterpret_cast<u32x2*>(b.Kt + (8 * dg + 2 * w) * kTP + 4 * kg) = lo;
        *reinterpret_cast<u32x2*>(b.Kt + (8 * dg + 2 * w + 1) * kTP + 4 * kg) = hi;
    }
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
        const int ci = tid + 256 * r4, row = ci >> 4, col = (ci & 15) * 8;
        *reinterpret_cast<u32x4*>(b.Qs + row * kQP + col) = bf16x8_to_f16x8(r.q[r4]);
    }
#pragma unroll
    for (int r2 = 0; r2 < 2; ++r2) {
        const int ci = tid + 256 * r2, row = ci >> 3, col = (ci & 7) * 8;
        *reinterpret_cast<u32x4*>(b.Ts + row * kTP + col) = r.t[r2];
        *reinterpret_cast<u32x4*>(b.Ps + row * kTP + col) = r.p[r2];
    }
    if (tid < 16) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            b.gs[4 * tid + u] = r.gb[u];
            b.egs[4 * tid + u] = __expf(r.gb[u]);
        }
    } else if (tid < 32) {
#pragma unroll
        for (int u = 0; u < 4; ++u) b.bs[4 * (tid - 16) + u] = r.gb[u];
    }
}

// A fragment of a 16-row block: row `row`, k-step covering columns [32*ks, 32*ks+32),
// slots j<4 -> column 32ks + 4G + j, slots j>=4 -> 32ks + 16 + 4G + (j-4).
__device__ __forceinline__ f16x8 afrag(const f16* base, int stride, int row, int ks, int G) {
    const f16* p = base + row * stride + 32 * ks + 4 * G;
    return cat(*reinterpret_cast<const f16x4*>(p), *reinterpret_cast<const f16x4*>(p + 16));
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

__global__ __launch_bounds__(256) void gla_scan_bf16_kernel(GlaLaunch g) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    ScanBuf* buf = reinterpret_cast<ScanBuf*>(smem);

    const int BH = g.BH;
    const int b = blockIdx.x;
    int bh, tile;
    if ((BH & 7) == 0) { bh = (b & 7) + 8 * (b >> 4); tile = (b >> 3) & 1; }   // both tiles of a head on one XCD
    else { bh = b >> 1; tile = b & 1; }
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int m = lane & 15, G = lane >> 4;
    const int col = tile * 64 + wave * 16 + m;
    const long long nch = (g.L + kC - 1) / kC;

    float* st = g.state + (long long)bh * kD * kD;
    f32x4 Mr[8];                                   // M[16kb + 4G + i][col]
#pragma unroll
    for (int kb = 0; kb < 8; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) Mr[kb][i] = st[(16 * kb + 4 * G + i) * kD + col];

    const bf16* vbh = static_cast<const bf16*>(g.v) + (long long)bh * g.L * kD;
    auto load_v = [&](long long c, bf16 (&vv)[16]) {
        const long long t0 = c * kC;
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const long long t = t0 + 16 * rb + 4 * G + i;
                vv[4 * rb + i] = t < g.L ? vbh[t * kD + col] : (bf16)0.f;
            }
    };

    StageRegs sr;
    bf16 vc[16], vn[16];
    stage_load(sr, g, bh, 0, tid);
    stage_store(sr, buf[0], tid);
    load_v(0, vc);
    __syncthreads();

    const float scale = g.scale;
    for (long long c = 0; c < nch; ++c) {
        const ScanBuf& B = buf[c & 1];
        const bool more = c + 1 < nch;
        if (more) {
            stage_load(sr, g, bh, c + 1, tid);
            load_v(c + 1, vn);
        }
        // K M0 and Q M0
        f16x8 bM[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) bM[ks] = bfrag(Mr[2 * ks], Mr[2 * ks + 1]);
        f32x4 KM[4], QM[4];
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
#pragma unroll
            for (int i = 0; i < 4; ++i) { KM[rb][i] = 0.f; QM[rb][i] = 0.f; }
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                KM[rb] = mfma16h(afrag(B.Ks, kQP, 16 * rb + m, ks, G), bM[ks], KM[rb]);
                QM[rb] = mfma16h(afrag(B.Qs, kQP, 16 * rb + m, ks, G), bM[ks], QM[rb]);
            }
        }
        // X = diag(beta) (V - diag(e^g) K M0)
        f32x4 X[4];
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 16 * rb + 4 * G + i;
                X[rb][i] = B.bs[t] * (bf2f(vc[4 * rb + i]) - B.egs[t] * KM[rb][i]);
            }
        f16x8 xb[2] = {bfrag(X[0], X[1]), bfrag(X[2], X[3])};
        // U = T X (T lower triangular: row blocks 0,1 only see k-step 0)
        f32x4 U[4];
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
#pragma unroll
            for (int i = 0; i < 4; ++i) U[rb][i] = 0.f;
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
                if (kt == 0 || rb >= 2) U[rb] = mfma16h(afrag(B.Ts, kTP, 16 * rb + m, kt, G), xb[kt], U[rb]);
        }
        const float gC = B.gs[kC - 1];
        f32x4 Us[4];
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
#pragma unroll
            for (int i = 0; i < 4; ++i) Us[rb][i] = U[rb][i] * __expf(gC - B.gs[16 * rb + 4 * G + i]);
        f16x8 ub[2] = {bfrag(U[0], U[1]), bfrag(U[2], U[3])};
        f16x8 usb[2] = {bfrag(Us[0], Us[1]), bfrag(Us[2], Us[3])};
        // O = diag(e^g) Q M0 + Pm U
        const long long t0 = c * kC;
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
            f32x4 PU;
#pragma unroll
            for (int i = 0; i < 4; ++i) PU[i] = 0.f;
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
                if (kt == 0 || rb >= 2) PU = mfma16h(afrag(B.Ps, kTP, 16 * rb + m, kt, G), ub[kt], PU);
            if (g.o) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = 16 * rb + 4 * G + i;
                    if (t0 + t < g.L) {
                        const float ov = scale * (B.egs[t] * QM[rb][i] + PU[i]);
                        const long long oi = ((long long)bh * g.L + t0 + t) * kD + col;
                        if (g.out_f32) static_cast<float*>(g.o)[oi] = ov;
                        else static_cast<bf16*>(g.o)[oi] = f2bf(ov);
                    }
                }
            }
        }
        // M = e^{g_C} M0 + K^T diag(e^{g_C - g}) U
        const float egC = __expf(gC);
#pragma unroll
        for (int kb = 0; kb < 8; ++kb) {
#pragma unroll
            for (int i = 0; i < 4; ++i) Mr[kb][i] *= egC;
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
                Mr[kb] = mfma16h(afrag(B.Kt, kTP, 16 * kb + m, kt, G), usb[kt], Mr[kb]);
        }
        if (more) {
            stage_store(sr, buf[(c + 1) & 1], tid);
#pragma unroll
            for (int i = 0; i < 16; ++i) vc[i] = vn[i];
        }
        __syncthreads();
    }
#pragma unroll
    for (int kb = 0; kb < 8; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) st[(16 * kb + 4 * G + i) * kD + col] = Mr[kb][i];
}

}  // namespace

size_t gla_bf16_workspace_bytes(int BH, long long L, int chunk) {
    (void)chunk;
    const long long nch = (L + kC - 1) / kC;
    return (size_t)BH * (size_t)nch * kChunkBytes;
}

hipError_t launch_gla_bf16(const GlaLaunch& g, hipStream_t stream) {
    if (g.BH == 0 || g.L == 0) return hipSuccess;
    if (g.d != kD || g.chunk != kC) return hipErrorInvalidValue;
    const long long nch = (g.L + kC - 1) / kC;
    if (g.ws_bytes < gla_bf16_workspace_bytes(g.BH, g.L, g.chunk)) return hipErrorInvalidValue;
    if ((long long)g.BH * nch > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL(gla_prep_bf16_kernel, dim3((unsigned)(g.BH * nch)), dim3(256), 0, stream, g,
                       (int)nch);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const size_t smem = 2 * sizeof(ScanBuf);   // > 64 KiB: raise the launch limit (current device)
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(gla_scan_bf16_kernel),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(gla_scan_bf16_kernel, dim3((unsigned)(g.BH * 2)), dim3(256), smem, stream, g);
    return hipGetLastError();
}

}  // namespace hta
