// gla_fwd.hip -- the bf16 GLA forward on MFMA (gfx950): chunk-parallel prep,
// then a chunk scan spread over 4 workgroups per head.
//
// Method: page "Kairos：面向物理 AI 的原生世界模型栈" (yingwang.github.io), section
// 二、方法, GLA paragraph and update equations, GatedDeltaNet reading:
//   S_t = alpha_t (S_{t-1} - beta_t (S_{t-1} k_t) k_t^T) + beta_t v_t k_t^T,  o_t = S_t q_t.
// State M = S^T (dk x dv). For a chunk of C = 64 tokens from M0, with g the
// inclusive cumulative sum of log alpha inside the chunk (the UT / WY form):
//   T = (I + A)^-1,  A = strictly-lower( diag(beta) (K K^T o e^{gp_i - g_j}) )
//   X = diag(beta) (V - diag(e^gp) (K M0)),   U = T X
//   O = diag(e^g) (Q M0) + Pm U,       Pm = tril(Q K^T o e^{g_i - g_j})
//   M = e^{g_C} M0 + K^T (diag(e^{g_C - g}) U)
// with gp = g (GatedDeltaNet) or the exclusive sum g_{i-1} (the printed update,
// whose erase term is not gated: only A and the K M0 term of X change).
//
// Precision and range. Inputs are bf16, every accumulation is fp32, and the
// operands the kernels build (K, Q, T, Pm, the state copy, X, U) are fp16,
// whose 11-bit significand keeps the chunk algebra about 8x closer to exact
// than bf16 operands. fp16 has a narrow range, so every fp16 operand carries a
// power-of-two scale (exact: it changes no rounding):
//   - per chunk, from the chunk's maxima (prep): K' = c K, Q' = c_q Q, T' = tau T,
//     with max |K'|, |Q'| in [8, 16) and max |T'| in [1/8, 1/4); then
//     Pm' = tril(Q' K'^T o e^{g_i - g_j}) = c c_q Pm is bounded by 128 * 16 * 16;
//     the reciprocals are folded into per-token factors;
//   - per value column, from the running maxima (scan): the state is kept as
//     sigma M and the values enter as sigma V, with sigma a power of two chosen
//     so that max(|sigma M|, |sigma V|) over the column stays in [1/16, 256]
//     (the recurrence is linear in (V, M0) column by column, so each column may
//     carry its own sigma; O and the final state are scaled back exactly).
// X and U then stay finite for any finite input as long as the keys keep the
// update from growing the state by more than the fp16 range allows within one
// chunk (with |k|_1 <= 11 -- any unit-norm key of 128 entries -- the fp16 X and
// U stay below 3.2e3 and 5.1e4). NaN and inf in the inputs propagate.
//
// Two kernels:
//   prep (one workgroup per chunk, all chunks in parallel): g; K K^T on
//     v_mfma_f32_32x32x16_bf16; A; T = (I + A)^-1 in fp32 by 16x16 blocks; the
//     chunk scales; and the chunk's operand block in exactly the LDS layout the
//     scan consumes (swizzles included): K', T', the per-token factors, then (with
//     an output) Q'. Optionally also copies the tokens' K and V into a ring slot (a
//     streamed frame).
//   scan (one workgroup per (batch, head, 32 value columns), chunks in order):
//     two state waves (16 columns each) run the recurrence with the state in MFMA
//     accumulator registers; two load waves stream the block and value tile of the
//     chunk after next into a three-stage LDS ring (direct global->LDS loads); two
//     output waves form Pm' from Q' and K', then the output from the state copy
//     and U' the state waves hand over in LDS. The four workgroups of a head run
//     on one XCD, so the block is fetched from HBM about once.
#include "device_common.h"
#include "gla_tiles.h"
#include "hta_internal.h"
#include "lds_dma.h"

namespace hta {

namespace {

using namespace glat;

// Operand block of one chunk (workspace and LDS stage share this layout).
constexpr int kFK = 0;                 // K' fp16 [64][128], chunks swizzled by swz64
constexpr int kFT = 16384;             // T' fp16 [64][64], chunks swizzled by swz32
constexpr int kFF = 24576;             // fp32 factors, [64] each:
constexpr int kFxa = 0;                //   beta                      (multiplies sigma V)
constexpr int kFxb = 64;               //   beta e^{gp} / c           (multiplies K' M0')
constexpr int kFud = 128;              //   e^{g_C - g} / (c tau)     (multiplies U' in the update)
constexpr int kFoe = 192;              //   e^{g} / c_q               (multiplies Q' M0' in O)
constexpr int kFg = 256;               //   g                         (the decay of Pm)
constexpr int kFsc = 320;              //   [0] e^{g_C}, [1] 1 / (c c_q tau) (multiplies Pm' U' in O)
constexpr int kFQ = 26112;             // Q' fp16 [64][128] (with an output)
constexpr int kFStateBytes = 26112;    // what the recurrence reads
constexpr int kFBlockBytes = 42496;    // ... and the output
static_assert(kFF + 6 * 256 == kFQ && kFQ + 16384 == kFBlockBytes, "block");
static_assert(kFQ % 256 == 0 && kFStateBytes % 1024 == 512 && kFBlockBytes % 1024 == 512, "layout");

constexpr int kKsP = kD + 8;           // padded K / Q row (bf16) of the prep
constexpr int kAsP = 68;               // padded A / T row (fp32) of the prep

// Power-of-two exponent k with m * 2^k in [2^target, 2^(target+1)); 0 for a zero
// or non-finite m (nothing to normalise), clamped to keep 2^k a normal float.
__device__ __forceinline__ int pow2_exp(float m, int target) {
    if (!(m > 0.f) || !(m < __builtin_huge_valf())) return 0;
    const int e = __builtin_amdgcn_frexp_expf(m) - 1;   // m in [2^e, 2^(e+1))
    return min(max(target - e, -120), 120);
}

// Largest |bf16| of eight, as the bit pattern of the magnitude (magnitudes of
// finite values order like the integers; inf and NaN sort above them).
__device__ __forceinline__ uint32_t bf16_absmax8(u32x4 w) {
    uint32_t m = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) m = max(m, max(w[j] & 0x7fffu, (w[j] >> 16) & 0x7fffu));
    return m;
}
__device__ __forceinline__ float bf16_bits_to_float(uint32_t b) {
    return b >= 0x7f80u ? 0.f : __uint_as_float(b << 16);   // inf / NaN: no scale
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x = max(x, (uint32_t)__shfl_xor((int)x, off, 64));
    return x;
}
__device__ __forceinline__ float wave_max_f32(float x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, 64));
    return x;
}

// Eight bf16 times a power of two, as eight fp16 (round to nearest even).
__device__ __forceinline__ u32x4 bf16x8_to_f16x8_scaled(u32x4 w, float s) {
    u32x4 r;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const f16 a = (f16)(__uint_as_float(w[j] << 16) * s);
        const f16 b = (f16)(__uint_as_float(w[j] & 0xffff0000u) * s);
        r[j] = (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
    }
    return r;
}

// Column order of the fp16 tiles (K', Q': 128 columns; T': 64): within each group
// of 32 columns, slot 8 G + j holds column 4 G + j for j < 4 and 16 + 4 G + (j - 4)
// for j >= 4 -- the contraction order in which a 16x16 MFMA accumulator pair is
// fed back as a B fragment (see bfrag) -- so that each A fragment of k-step ks,
// lane group G is the single 16-byte chunk 4 ks + G of its row.
__device__ __forceinline__ int slot32(int c) {
    const int x = c & 31;
    return (c & ~31) | (x < 16 ? 8 * (x >> 2) + (x & 3) : 8 * ((x - 16) >> 2) + 4 + (x & 3));
}
// Byte offset of element (row, column) in a K' / Q' tile (256-byte rows, chunks
// swizzled by swz64) and in a T' tile (128-byte rows, swz32).
__device__ __forceinline__ int offKp(int row, int col) {
    const int p = slot32(col);
    return row * 256 + 16 * ((p >> 3) ^ swz64(row)) + 2 * (p & 7);
}
__device__ __forceinline__ int offTp(int row, int col) {
    const int p = slot32(col);
    return row * 128 + 16 * ((p >> 3) ^ swz32(row)) + 2 * (p & 7);
}
// A fragment of rows 16-block `row` (lane's row), k-step ks, lane group G.
__device__ __forceinline__ f16x8 fragK(const char* base, int row, int ks, int G) {
    return *reinterpret_cast<const f16x8*>(base + row * 256 + 16 * ((4 * ks + G) ^ swz64(row)));
}
__device__ __forceinline__ f16x8 fragT(const char* base, int row, int kt, int G) {
    return *reinterpret_cast<const f16x8*>(base + row * 128 + 16 * ((4 * kt + G) ^ swz32(row)));
}
// K'^T fragment for d-block kb, k-step kt (tokens 32 kt + 4 G + j, + 16) by two
// transposed reads: source lane 4j + a addresses token row 32 kt + 4 G + j,
// columns 16 kb + 4 a .. +3 (four adjacent slots); lane 4 a + b receives column b
// of rows j = 0..3.
__device__ __forceinline__ f16x8 fragKt(const char* base, int kb, int kt, int lane) {
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    const int G = lane >> 4, sl = lane & 15, j = sl >> 2, a = sl & 3;
    const int t0 = 32 * kt + 4 * G + j;
    const int col = 16 * kb + 4 * a;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + offKp(t0, col)));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + offKp(t0 + 16, col)));
    return cat(__builtin_bit_cast(f16x4, lo), __builtin_bit_cast(f16x4, hi));
}

// ------------------------------------------------------------------ prep

// One workgroup per chunk. Phases, separated by barriers:
//   1. loads: alpha, beta (wave 0), K (and Q) rows, K kept in LDS as bf16; the
//      chunk maxima of |k| (|q|); the decay prefix sums (wave 0);
//   2. K' (Q') written to the block; K K^T on MFMA, one 32x32 block per wave;
//   3. A into LDS;
//   4. T = (I + A)^-1 in fp32 by 16x16 blocks: each wave inverts one diagonal block
//      by forward substitution, then the blocks below the diagonal follow in three
//      levels of products, T_ik = -T_ii sum_{k <= j < i} A_ij T_jk (from (I + A) T = I);
//   5. max |T|, T' staged in fp16 and copied out; the per-token factors.
template <bool OUT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4)))
void gla_prep2_kernel(GlaLaunch g, int nch, int stride) {
    __shared__ __attribute__((aligned(16))) bf16 Ks[kC * kKsP];   // K; then T (fp32)
    __shared__ __attribute__((aligned(16))) float As[kC * kAsP];  // Q (bf16); then A; then T' staging
    __shared__ float gs[kC];
    __shared__ float gps[kC];   // decay exponent of the erase path (g, or g_{i-1} for the printed form)
    __shared__ float bs[kC];
    __shared__ float red[3][4]; // per-wave maxima: |k|, |q|, |T|

    const int cid = blockIdx.x;
    const int bh = cid / nch, c = cid - bh * nch;
    const long long t0 = (long long)c * kC;
    const int n = (int)min((long long)kC, g.L - t0);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const bf16* kp = static_cast<const bf16*>(g.k) + ((long long)bh * g.L + t0) * kD;
    const bf16* qp = static_cast<const bf16*>(g.q) + ((long long)bh * g.L + t0) * kD;
    char* blk = static_cast<char*>(g.ws) + (size_t)cid * (size_t)stride;

    float alpha_t = 1.f, beta_t = 0.f;
    if (wave == 0 && lane < n) {
        alpha_t = g.alpha[(long long)bh * g.L + t0 + lane];
        beta_t = g.beta[(long long)bh * g.L + t0 + lane];
    }
    u32x4 kv[4], qv[4], vv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int ci = tid + 256 * r, row = ci >> 4, cc = ci & 15;
        kv[r] = u32x4{0u, 0u, 0u, 0u};
        qv[r] = u32x4{0u, 0u, 0u, 0u};
        if (row < n) {
            kv[r] = *reinterpret_cast<const u32x4*>(kp + (long long)row * kD + 8 * cc);
            if (OUT) qv[r] = *reinterpret_cast<const u32x4*>(qp + (long long)row * kD + 8 * cc);
            if (g.ring_v)
                vv[r] = *reinterpret_cast<const u32x4*>(static_cast<const bf16*>(g.v) +
                                                        ((long long)bh * g.L + t0 + row) * kD + 8 * cc);
        }
    }
    uint32_t mk = 0, mq = 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int ci = tid + 256 * r, row = ci >> 4, cc = ci & 15;
        *reinterpret_cast<u32x4*>(Ks + row * kKsP + 8 * cc) = kv[r];
        if (OUT) *reinterpret_cast<u32x4*>(reinterpret_cast<bf16*>(As) + row * kKsP + 8 * cc) = qv[r];
        mk = max(mk, bf16_absmax8(kv[r]));
        if (OUT) mq = max(mq, bf16_absmax8(qv[r]));
        if (g.ring_k && row < n) {   // the chunk's K and V rows into the ring slot, unchanged
            const long long ro = (long long)bh * g.ring_bh + g.ring_off + (t0 + row) * kD + 8 * cc;
            *reinterpret_cast<u32x4*>(static_cast<bf16*>(g.ring_k) + ro) = kv[r];
            *reinterpret_cast<u32x4*>(static_cast<bf16*>(g.ring_v) + ro) = vv[r];
        }
    }
    mk = wave_max_u32(mk);
    if (OUT) mq = wave_max_u32(mq);
    if (lane == 0) {
        red[0][wave] = bf16_bits_to_float(mk);
        red[1][wave] = bf16_bits_to_float(mq);
    }
    if (wave == 0) {
        // inclusive prefix sum of log(alpha) over the chunk (alpha = 1 past the end)
        float la = 0.f;
        if (lane < n) {
            const float lg = logf(alpha_t);
            la = (lg < kLogFloor) ? kLogFloor : lg;   // NaN passes through
        }
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float y = __shfl_up(la, off, 64);
            if (lane >= off) la += y;
        }
        const float prev = __shfl_up(la, 1, 64);
        gs[lane] = la;
        gps[lane] = g.form ? (lane == 0 ? 0.f : prev) : la;
        bs[lane] = beta_t;
    }
    __syncthreads();

    const int ek = pow2_exp(fmaxf(fmaxf(red[0][0], red[0][1]), fmaxf(red[0][2], red[0][3])), 3);
    const int eq = OUT ? pow2_exp(fmaxf(fmaxf(red[1][0], red[1][1]), fmaxf(red[1][2], red[1][3])), 3) : 0;
    {
        // stored chunk s of a row holds slots 8 s .. 8 s + 7: columns 32 (s / 4) + 4 (s % 4)
        // .. +3 and 32 (s / 4) + 16 + 4 (s % 4) .. +3 (two 8-byte pieces of the LDS copy)
        const float ck = __builtin_ldexpf(1.f, ek), cq = __builtin_ldexpf(1.f, eq);
        const bf16* Qs = reinterpret_cast<const bf16*>(As);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int ci = tid + 256 * r, row = ci >> 4, sch = ci & 15;
            const int c0 = 32 * (sch >> 2) + 4 * (sch & 3);
            const int dst = row * 256 + 16 * (sch ^ swz64(row));
            const u32x2 k0 = *reinterpret_cast<const u32x2*>(Ks + row * kKsP + c0);
            const u32x2 k1 = *reinterpret_cast<const u32x2*>(Ks + row * kKsP + c0 + 16);
            *reinterpret_cast<u32x4*>(blk + kFK + dst) =
                bf16x8_to_f16x8_scaled(u32x4{k0[0], k0[1], k1[0], k1[1]}, ck);
            if (OUT) {
                const u32x2 q0 = *reinterpret_cast<const u32x2*>(Qs + row * kKsP + c0);
                const u32x2 q1 = *reinterpret_cast<const u32x2*>(Qs + row * kKsP + c0 + 16);
                *reinterpret_cast<u32x4*>(blk + kFQ + dst) =
                    bf16x8_to_f16x8_scaled(u32x4{q0[0], q0[1], q1[0], q1[1]}, cq);
            }
        }
    }

    // K K^T, one 32x32 block per wave (the upper one stays zero).
    const int mb = wave >> 1, nb = wave & 1;
    const int nn = lane & 31, h = lane >> 5;
    f32x16 kk;
#pragma unroll
    for (int i = 0; i < 16; ++i) kk[i] = 0.f;
    if (mb >= nb) {
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            const bf16x8 ka = *reinterpret_cast<const bf16x8*>(Ks + (mb * 32 + nn) * kKsP + 16 * ks + 8 * h);
            const bf16x8 kb = *reinterpret_cast<const bf16x8*>(Ks + (nb * 32 + nn) * kKsP + 16 * ks + 8 * h);
            kk = mfma32(ka, kb, kk);
        }
    }
    __syncthreads();   // Q (in the A buffer) converted by every wave
    {
        const int j = nb * 32 + nn;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int i = mb * 32 + 8 * (e >> 2) + 4 * h + (e & 3);
            const float deca = (j < i) ? __expf(gps[i] - gs[j]) : 0.f;
            As[i * kAsP + j] = (j < i) ? bs[i] * deca * kk[e] : 0.f;
        }
    }
    __syncthreads();

    // Diagonal block kb = wave of T by forward substitution: lane (column c, sub)
    // keeps x_r for the block's rows r = 4 m + sub (entries not yet solved are 0,
    // and so is A on and above the diagonal, so every product term is safe).
    float* Ts = reinterpret_cast<float*>(Ks);   // T, fp32 [64][kAsP]
    {
        const int kb = wave, cl = lane >> 2, sub = lane & 3;
        const float* Ab = As + 16 * kb * kAsP + 16 * kb;
        float x[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float* ar = Ab + i * kAsP + sub;
            float part = (ar[0] * x[0] + ar[4] * x[1]) + (ar[8] * x[2] + ar[12] * x[3]);
            part += quad_xor1(part);   // sum over the quad's four lanes, in registers
            part += quad_xor2(part);
            const float xi = (i == cl ? 1.f : 0.f) - part;
            if ((i & 3) == sub) x[i >> 2] = xi;
        }
        __syncthreads();   // every wave's K K^T read of K is done (same buffer)
#pragma unroll
        for (int mm = 0; mm < 4; ++mm) Ts[(16 * kb + 4 * mm + sub) * kAsP + 16 * kb + cl] = x[mm];
    }
    __syncthreads();
    // Blocks (k + d, k) at level d, wave k: S = sum_j A_ij T_jk, then T_ik = -T_ii S
    // (S staged in the block's own slot: each wave reads it back before overwriting).
    {
        const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
        const int nl = lane & 15, gq = lane >> 4;
#pragma unroll
        for (int d = 1; d < 4; ++d) {
            if (wave < 4 - d) {
                const int k = wave, i = k + d;
                f32x4 sacc = zero4;
                for (int j = k; j < i; ++j)
                    sacc = mm16f(As + 16 * i * kAsP + 16 * j, kAsP, Ts + 16 * j * kAsP + 16 * k, kAsP,
                                 sacc, lane);
                float* Tik = Ts + 16 * i * kAsP + 16 * k;
#pragma unroll
                for (int r = 0; r < 4; ++r) Tik[(4 * gq + r) * kAsP + nl] = sacc[r];
                const f32x4 t = mm16f(Ts + 16 * i * kAsP + 16 * i, kAsP, Tik, kAsP, zero4, lane);
#pragma unroll
                for (int r = 0; r < 4; ++r) Tik[(4 * gq + r) * kAsP + nl] = -t[r];
            }
            __syncthreads();
        }
    }
    // max |T| over the lower triangle (the diagonal is 1), then T' = tau T in fp16,
    // staged in the block layout in the A buffer and copied out.
    {
        float tmax = 0.f;
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int q = tid + 256 * r, i = q >> 3, j0 = (q & 7) * 8;
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (j0 + u <= i) tmax = fmaxf(tmax, fabsf(Ts[i * kAsP + j0 + u]));
        }
        tmax = wave_max_f32(tmax);
        if (lane == 0) red[2][wave] = tmax;
    }
    __syncthreads();
    const int et = pow2_exp(fmaxf(fmaxf(red[2][0], red[2][1]), fmaxf(red[2][2], red[2][3])), -3);
    char* stT = reinterpret_cast<char*>(As);
    {
        const float tau = __builtin_ldexpf(1.f, et);
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int q = tid + 256 * r, i = q >> 3, j0 = (q & 7) * 8;
            const float* tr = Ts + i * kAsP + j0;
            f16x8 h8;
#pragma unroll
            for (int u = 0; u < 8; ++u) h8[u] = (f16)((j0 + u <= i) ? tr[u] * tau : 0.f);
            *reinterpret_cast<f16x4*>(stT + offTp(i, j0)) = f16x4{h8[0], h8[1], h8[2], h8[3]};
            *reinterpret_cast<f16x4*>(stT + offTp(i, j0 + 4)) = f16x4{h8[4], h8[5], h8[6], h8[7]};
        }
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int q = tid + 256 * r;
        *reinterpret_cast<u32x4*>(blk + kFT + 16 * q) = *reinterpret_cast<const u32x4*>(stT + 16 * q);
    }
    if (wave == 0) {
        float* f = reinterpret_cast<float*>(blk + kFF);
        const float la = gs[lane], gC = gs[kC - 1], b = bs[lane];
        f[kFxa + lane] = b;
        f[kFxb + lane] = b * __builtin_ldexpf(__expf(gps[lane]), -ek);
        f[kFud + lane] = __builtin_ldexpf(__expf(gC - la), -(ek + et));
        f[kFoe + lane] = __builtin_ldexpf(__expf(la), -eq);
        f[kFg + lane] = la;
        f[kFsc + lane] = lane == 0 ? __expf(gC) : (lane == 1 ? __builtin_ldexpf(1.f, -(ek + eq + et)) : 0.f);
    }
}

// ------------------------------------------------------------------ scan

// LDS of the scan for NCG 16-column groups per workgroup: an NST-stage ring
// (operand block + value tile), then the hand-over from the state waves to the
// output waves -- the state copy M0' and U', already rounded to the fp16 B
// fragments the products consume (fragment k of lane l of column group w at
// ((w * nfrag + k) * 64 + l) * 16), and 1/sigma of their columns.
template <int NCG, int NW, int NST>
struct Scan3 {
    static constexpr int kVRow = 32 * NCG;                 // bytes per token row of the V tile
    static constexpr int kOffV = kFBlockBytes;
    static constexpr int kStage = kFBlockBytes + kC * kVRow;
    static constexpr int kNStage = NST;
    static constexpr int kXm = kNStage * kStage;
    static constexpr int kXu = kXm + NCG * 4 * 1024;
    static constexpr int kSm = kXu + NCG * 2 * 1024;
    static constexpr int kSu = kSm + NCG * 64;
    static constexpr int kLds = kSu + NCG * 64;
    static constexpr int kThreads = 64 * NW;   // NW waves in all
};

// V tile: token row t holds the workgroup's 16 NCG columns; its 16-byte chunk c
// sits in slot c ^ vswz(t) (with two column groups, rows 4..7 mod 8 swap halves,
// so the transposed reads of the two 32-lane halves of a wave use disjoint banks).
template <int NCG>
__device__ __forceinline__ int vswz(int t) { return NCG == 2 ? 2 * ((t >> 2) & 1) : 0; }
template <int NCG>
__device__ __forceinline__ int offV(int t, int col) {
    return t * 32 * NCG + 16 * ((col >> 3) ^ vswz<NCG>(t)) + 2 * (col & 7);
}

// Max over the four lanes l, l^16, l^32, l^48 (one value column of the state).
__device__ __forceinline__ float colmax(float x) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
    r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float absmax_state(const f32x4 (&M)[8]) {
    float a = 0.f, b = 0.f;
#pragma unroll
    for (int kb = 0; kb < 8; kb += 2) {
        a = fmaxf(a, fmaxf(fmaxf(fabsf(M[kb][0]), fabsf(M[kb][1])), fmaxf(fabsf(M[kb][2]), fabsf(M[kb][3]))));
        b = fmaxf(b, fmaxf(fmaxf(fabsf(M[kb + 1][0]), fabsf(M[kb + 1][1])),
                           fmaxf(fabsf(M[kb + 1][2]), fabsf(M[kb + 1][3]))));
    }
    return fmaxf(a, b);
}

// Loads one load wave issues per chunk: the first `nbytes` of the block in 1 KiB
// pieces and the value tile (2 NCG pieces), dealt round-robin over ND waves.
template <int NCG, int ND, int NBYTES>
struct ChunkLoads {
    static constexpr int kPieces = (NBYTES + 1023) / 1024 + 2 * NCG;
    static constexpr int count(int w) { return (kPieces - w + ND - 1) / ND; }
};

// Enqueue pieces [first, last) of this wave's share of chunk c's block (the first
// NBYTES) and the workgroup's value tile into an LDS stage; lw is the issuing wave
// among the ND load waves, which take the 1 KiB pieces round-robin.
template <int NCG, int ND, int NBYTES>
__device__ __forceinline__ void issue_chunk3(char* stage, const GlaLaunch& g, int bh, int tile,
                                             long long c, long long nch, int stride, int lw, int lane,
                                             int first, int last) {
    constexpr int n16 = NBYTES >> 4, nblk = (n16 + 63) / 64;
    const char* blk = static_cast<const char*>(g.ws) + (size_t)((long long)bh * nch + c) * (size_t)stride;
    const long long t0 = c * kC;
    const int n = (int)min((long long)kC, g.L - t0);
    const bf16* vb = static_cast<const bf16*>(g.v) + ((long long)bh * g.L + t0) * kD + tile * 16 * NCG;
    for (int i = lw + first * ND; i < nblk + 2 * NCG && i < lw + last * ND; i += ND) {
        if (i < nblk) {
            const int p = 64 * i + lane;
            if (p < n16) dma16p(blk + 16 * p, stage + 1024 * i);
        } else {
            const int p = 64 * (i - nblk) + lane;
            const int tok = p / (2 * NCG), sl = p % (2 * NCG);
            const int cc = sl ^ vswz<NCG>(tok);
            dma16p(vb + (long long)min(tok, n - 1) * kD + 8 * cc, stage + kFBlockBytes + 1024 * (i - nblk));
        }
    }
}

// This wave's loads of the current chunk have landed: with the next chunk's loads
// (CNT of them) issued after them, wait until only those are outstanding.
template <int NCG, int ND, int NBYTES>
__device__ __forceinline__ void wait_chunk3(int lw, bool next_issued) {
    using CL = ChunkLoads<NCG, ND, NBYTES>;
    if (!next_issued) { wait_vmcnt<0>(); return; }
    switch (lw) {
        case 0: wait_vmcnt<CL::count(0)>(); break;
        case 1: wait_vmcnt<CL::count(1)>(); break;
        case 2: wait_vmcnt<CL::count(2)>(); break;
        case 3: wait_vmcnt<CL::count(3)>(); break;
        case 4: wait_vmcnt<CL::count(4)>(); break;
        default: wait_vmcnt<CL::count(5)>(); break;
    }
}

// One workgroup per (batch, head, 16 NCG value columns); waves:
//   0 .. NCG-1       state waves (column group cg = wave): K' M0', X, U' = T' X
//                    and the update of the scaled state; they publish M0' and U'
//                    (and 1/sigma of their columns) to LDS and touch no global
//                    memory inside the loop;
//   NCG ..           with an output (OUTK 1: fp32, 2: bf16), two output waves: for
//                    token blocks {0, 3} or {1, 2} (equal MFMA counts) they form
//                    Pm' = tril(Q' K'^T o e^{g_i - g_j}) and Q' M0', then
//                    O = (e^g / c_q) Q' M0' / sigma + Pm' U' / (c c_q tau sigma),
//                    stored 16 bytes per lane;
//   the last ND      load waves: chunk c + NST - 1 into the ring while chunk c is
//                    processed (a wave's loads go out slowly, so several waves
//                    share them).
// Barriers per chunk: B1 (chunk c staged, M0' published) and, with an output,
// B2 (U' published).
template <int NCG, int ND, int NST, int OUTK>
__global__ __launch_bounds__((Scan3<NCG, NCG + (OUTK ? 2 : 0) + ND, NST>::kThreads))
__attribute__((amdgpu_waves_per_eu(1, 2)))
void gla_scan3_kernel(GlaLaunch g, int stride) {
    using Ly = Scan3<NCG, NCG + (OUTK ? 2 : 0) + ND, NST>;
    extern __shared__ __attribute__((aligned(1024))) char smem[];
    constexpr int NT = 8 / NCG;                  // workgroups per head
    constexpr int NBYTES = OUTK ? kFBlockBytes : kFStateBytes;

    const int b = blockIdx.x;
    int bh, tile;
    if ((g.BH & 7) == 0) {   // the head's NT workgroups on one XCD (dispatch is round-robin over 8)
        const int x = b & 7, j = b >> 3;
        bh = x + 8 * (j / NT);
        tile = j % NT;
    } else {
        bh = b / NT;
        tile = b % NT;
    }
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int m = lane & 15, G = lane >> 4;
    const long long nch = (g.L + kC - 1) / kC;
    f16x8* xm = reinterpret_cast<f16x8*>(smem + Ly::kXm);
    f16x8* xu = reinterpret_cast<f16x8*>(smem + Ly::kXu);
    float* sM = reinterpret_cast<float*>(smem + Ly::kSm);
    float* sU = reinterpret_cast<float*>(smem + Ly::kSu);
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
    auto stage_of = [&](long long c) { return smem + (int)(c % Ly::kNStage) * Ly::kStage; };

    if (wave < NCG) {
        const int cg = wave;
        const int col = tile * 16 * NCG + 16 * cg + m;
        float* st = g.state + (long long)bh * kD * kD;
        f32x4 Ms[8];   // sigma * M[16 kb + 4 G + i][col]
#pragma unroll
        for (int kb = 0; kb < 8; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i) Ms[kb][i] = st[(16 * kb + 4 * G + i) * kD + col];
        float mS = colmax(absmax_state(Ms));
        int es = pow2_exp(mS, 4);                 // sigma = 2^es
        {
            const float s = __builtin_ldexpf(1.f, es);
#pragma unroll
            for (int kb = 0; kb < 8; ++kb) Ms[kb] *= s;
            mS *= s;
        }
        f16x8 bM[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            bM[ks] = bfrag(Ms[2 * ks], Ms[2 * ks + 1]);
            if (OUTK) xm[(cg * 4 + ks) * 64 + lane] = bM[ks];
        }
        if (OUTK && G == 0) sM[cg * 16 + m] = __builtin_ldexpf(1.f, -es);
        for (long long c = 0; c < nch; ++c) {
            __syncthreads();   // B1: chunk c staged; M0' published
            const char* S = stage_of(c);
            const float* fa = reinterpret_cast<const float*>(S + kFF);
            // K' fragments and V first; K' M0' goes out on the current scale while the
            // values' maximum is taken on the vector unit.
            f16x8 kf[4][4];
#pragma unroll
            for (int rb = 0; rb < 4; ++rb)
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) kf[rb][ks] = fragK(S + kFK, 16 * rb + m, ks, G);
            // V[16rb + 4G + i][col], i = 0..3, by one transposed read per row block:
            // source lane 4j + a addresses token 16rb + 4G + j, columns 16cg + 4a .. +3.
            bf16x4 v4[4];
            {
                typedef short s16x4 __attribute__((ext_vector_type(4)));
                typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
                const int j = m >> 2, a = m & 3;
#pragma unroll
                for (int rb = 0; rb < 4; ++rb) {
                    const int t = 16 * rb + 4 * G + j;
                    v4[rb] = __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_s16x4*)(S + Ly::kOffV + offV<NCG>(t, 16 * cg + 4 * a))));
                }
            }
            f32x4 KM[4];
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) {
                KM[rb] = zero4;
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) KM[rb] = mfma16h(kf[rb][ks], bM[ks], KM[rb]);
            }
            float vf[4][4];
            float vm = 0.f;
#pragma unroll
            for (int rb = 0; rb < 4; ++rb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    vf[rb][i] = bf2f(v4[rb][i]);
                    vm = fmaxf(vm, fabsf(vf[rb][i]));
                }
            // The column's scale: the values and the state together in [1/16, 256]
            // (rarely violated: then rescale and redo K' M0').
            {
                const float r = fmaxf(mS, __builtin_ldexpf(colmax(vm), es));
                if (r > 256.f || (r > 0.f && r < 0.0625f)) {
                    const int d = pow2_exp(r, 4);
                    const float s = __builtin_ldexpf(1.f, d);
                    es += d;
                    mS *= s;
#pragma unroll
                    for (int kb = 0; kb < 8; ++kb) Ms[kb] *= s;
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks) bM[ks] = bfrag(Ms[2 * ks], Ms[2 * ks + 1]);
#pragma unroll
                    for (int rb = 0; rb < 4; ++rb) KM[rb] *= s;
                }
            }
            const float sg = __builtin_ldexpf(1.f, es);
            // sigma X = beta (sigma V) - (beta e^gp / c) K' M0'
            f32x4 X[4];
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) {
                const f32x4 xa4 = *reinterpret_cast<const f32x4*>(fa + kFxa + 16 * rb + 4 * G);
                const f32x4 xb4 = *reinterpret_cast<const f32x4*>(fa + kFxb + 16 * rb + 4 * G);
#pragma unroll
                for (int i = 0; i < 4; ++i) X[rb][i] = xa4[i] * (sg * vf[rb][i]) - xb4[i] * KM[rb][i];
            }
            const f16x8 xb[2] = {bfrag(X[0], X[1]), bfrag(X[2], X[3])};
            // U' = T' X (T lower triangular: row blocks 0,1 only see k-step 0)
            f32x4 U[4];
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) {
                U[rb] = mfma16h(fragT(S + kFT, 16 * rb + m, 0, G), xb[0], zero4);
                if (rb >= 2) U[rb] = mfma16h(fragT(S + kFT, 16 * rb + m, 1, G), xb[1], U[rb]);
            }
            if (OUTK) {
                xu[(cg * 2 + 0) * 64 + lane] = bfrag(U[0], U[1]);
                xu[(cg * 2 + 1) * 64 + lane] = bfrag(U[2], U[3]);
                if (G == 0) sU[cg * 16 + m] = __builtin_ldexpf(1.f, -es);
            }
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) {
                const f32x4 ud4 = *reinterpret_cast<const f32x4*>(fa + kFud + 16 * rb + 4 * G);
#pragma unroll
                for (int i = 0; i < 4; ++i) U[rb][i] *= ud4[i];
            }
            const f16x8 usb[2] = {bfrag(U[0], U[1]), bfrag(U[2], U[3])};
            // K'^T fragments (transposed reads of the stage) ahead of the barrier
            f16x8 kt[8][2];
#pragma unroll
            for (int kb = 0; kb < 8; ++kb) {
                kt[kb][0] = fragKt(S + kFK, kb, 0, lane);
                kt[kb][1] = fragKt(S + kFK, kb, 1, lane);
            }
            const float egC = fa[kFsc];
            if (OUTK) __syncthreads();   // B2: U' published; the output waves are done with M0'
            // sigma M = e^{g_C} sigma M0 + K'^T diag(e^{g_C - g} / (c tau)) U'
#pragma unroll
            for (int kb = 0; kb < 8; ++kb) {
                Ms[kb] *= egC;
                Ms[kb] = mfma16h(kt[kb][0], usb[0], Ms[kb]);
                Ms[kb] = mfma16h(kt[kb][1], usb[1], Ms[kb]);
            }
            mS = colmax(absmax_state(Ms));
            if (mS > 256.f) {   // the state outgrew its scale: lower sigma before the fp16 copy
                const int d = pow2_exp(mS, 4);
                const float s = __builtin_ldexpf(1.f, d);
                es += d;
                mS *= s;
#pragma unroll
                for (int kb = 0; kb < 8; ++kb) Ms[kb] *= s;
            }
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                bM[ks] = bfrag(Ms[2 * ks], Ms[2 * ks + 1]);
                if (OUTK) xm[(cg * 4 + ks) * 64 + lane] = bM[ks];
            }
            if (OUTK && G == 0) sM[cg * 16 + m] = __builtin_ldexpf(1.f, -es);
        }
        const float inv = __builtin_ldexpf(1.f, -es);
#pragma unroll
        for (int kb = 0; kb < 8; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i) st[(16 * kb + 4 * G + i) * kD + col] = Ms[kb][i] * inv;
        return;
    }
    const int hw = wave - NCG;
    if (OUTK && hw < 2) {
        // Output waves: token blocks rbs[0], rbs[1]. Both products are formed
        // transposed: Pm'^T = K' Q'^T (its accumulator tiles become the B fragments of
        // U'^T Pm'^T as they are) and O^T = M0'^T Q'^T + U'^T Pm'^T, so lane (m, G)
        // ends up holding O[16 rb + m][16 cg + 4G + i], four adjacent columns of one token.
        const int rbs[2] = {hw == 0 ? 0 : 1, hw == 0 ? 3 : 2};
        const float scale = g.scale;
        for (long long c = 0; c < nch; ++c) {
            __syncthreads();   // B1
            const char* S = stage_of(c);
            const float* fa = reinterpret_cast<const float*>(S + kFF);
            f16x8 pmb[2][2];   // [r][kt]: B fragments of Pm'^T for token block rbs[r]
            f32x4 QM[2][NCG];
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                const int rb = rbs[r];
                f16x8 qf[4];
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) qf[ks] = fragK(S + kFQ, 16 * rb + m, ks, G);
                // Pm'^T blocks (cb, rb), cb <= rb: lane (m, G) gets Pm'[16 rb + m][16 cb + 4G + i]
                const int i_tok = 16 * rb + m;
                const float gi = fa[kFg + i_tok];
                f32x4 pt[4];
#pragma unroll
                for (int cb = 0; cb < 4; ++cb) {
                    pt[cb] = zero4;
                    if (cb <= rb) {
#pragma unroll
                        for (int ks = 0; ks < 4; ++ks)
                            pt[cb] = mfma16h(fragK(S + kFK, 16 * cb + m, ks, G), qf[ks], pt[cb]);
                        const f32x4 gj = *reinterpret_cast<const f32x4*>(fa + kFg + 16 * cb + 4 * G);
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int j_tok = 16 * cb + 4 * G + i;
                            pt[cb][i] = (j_tok <= i_tok) ? pt[cb][i] * __expf(gi - gj[i]) : 0.f;
                        }
                    }
                }
                pmb[r][0] = bfrag(pt[0], pt[1]);
                pmb[r][1] = bfrag(pt[2], pt[3]);
#pragma unroll
                for (int cg = 0; cg < NCG; ++cg) {
                    QM[r][cg] = zero4;
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks)
                        QM[r][cg] = mfma16h(xm[(cg * 4 + ks) * 64 + lane], qf[ks], QM[r][cg]);
                }
            }
            f32x4 smi[NCG];
#pragma unroll
            for (int cg = 0; cg < NCG; ++cg) smi[cg] = *reinterpret_cast<const f32x4*>(sM + cg * 16 + 4 * G);
            __syncthreads();   // B2
            const long long t0 = c * kC;
            const float p = scale * fa[kFsc + 1];
#pragma unroll
            for (int cg = 0; cg < NCG; ++cg) {
                const f16x8 ub0 = xu[(cg * 2 + 0) * 64 + lane], ub1 = xu[(cg * 2 + 1) * 64 + lane];
                const f32x4 sui = *reinterpret_cast<const f32x4*>(sU + cg * 16 + 4 * G);
#pragma unroll
                for (int r = 0; r < 2; ++r) {
                    const int rb = rbs[r];
                    f32x4 PU = mfma16h(ub0, pmb[r][0], zero4);
                    if (rb >= 2) PU = mfma16h(ub1, pmb[r][1], PU);
                    const int tok = 16 * rb + m;
                    const float e = scale * fa[kFoe + tok];
                    f32x4 ov;
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        ov[i] = (e * smi[cg][i]) * QM[r][cg][i] + (p * sui[i]) * PU[i];
                    if (t0 + tok < g.L) {
                        const long long off = ((long long)bh * g.L + t0 + tok) * kD + tile * 16 * NCG +
                                              16 * cg + 4 * G;
                        if (OUTK == 1) {
                            *reinterpret_cast<f32x4*>(static_cast<float*>(g.o) + off) = ov;
                        } else {
                            bf16x4 ob;
#pragma unroll
                            for (int i = 0; i < 4; ++i) ob[i] = (bf16)ov[i];
                            *reinterpret_cast<bf16x4*>(static_cast<bf16*>(g.o) + off) = ob;
                        }
                    }
                }
            }
        }
        return;
    }
    // Load waves: chunks 0 .. NST-2 up front, then chunk c + NST - 1 once chunk c is
    // staged (its stage last held chunk c - 1, which every wave finished before B1);
    // with an output, half of the pieces after B1 and half after B2, so that neither
    // barrier waits for the slow issue of all of them.
    const int lw = OUTK ? hw - 2 : hw;
    constexpr int kAll = 1 << 20, kHalf = (ChunkLoads<NCG, ND, NBYTES>::count(0) + 1) / 2;
    for (int p = 0; p < NST - 1 && p < nch; ++p)
        issue_chunk3<NCG, ND, NBYTES>(stage_of(p), g, bh, tile, p, nch, stride, lw, lane, 0, kAll);
    for (long long c = 0; c < nch; ++c) {
        // with three stages, chunk c + 1's loads (issued after chunk c's) may stay in flight
        wait_chunk3<NCG, ND, NBYTES>(lw, NST == 3 && c + 1 < nch);
        __syncthreads();   // B1
        const long long cn = c + NST - 1;
        if (cn < nch)
            issue_chunk3<NCG, ND, NBYTES>(stage_of(cn), g, bh, tile, cn, nch, stride, lw, lane, 0,
                                          OUTK ? kHalf : kAll);
        if (OUTK) {
            __syncthreads();   // B2
            if (cn < nch)
                issue_chunk3<NCG, ND, NBYTES>(stage_of(cn), g, bh, tile, cn, nch, stride, lw, lane,
                                              kHalf, kAll);
        }
    }
}

// Two shapes of the scan: the whole chip (one 16-column group per workgroup, eight
// workgroups per head, three stages, five load waves), and a narrow one for running
// beside other work (four column groups per workgroup, two per head, two stages).
template <int NCG, int ND, int NST>
struct ScanShape {
    static constexpr int kNcg = NCG, kNd = ND, kNst = NST;
    template <int OUTK>
    using Ly = Scan3<NCG, NCG + (OUTK ? 2 : 0) + ND, NST>;
    static_assert(Ly<1>::kLds <= 160 * 1024, "scan LDS exceeds one CU");
    static_assert(ND <= 6 && ChunkLoads<NCG, ND, kFBlockBytes>::count(0) < 64, "vmcnt range");
};
using WideScan = ScanShape<1, 5, 3>;
using NarrowScan = ScanShape<4, 2, 2>;

template <class SH, int OUTK>
hipError_t launch_scan3(const GlaLaunch& g, int stride, hipStream_t stream) {
    using Ly = typename SH::template Ly<OUTK>;
    auto kern = gla_scan3_kernel<SH::kNcg, SH::kNd, SH::kNst, OUTK>;
    const void* fn = reinterpret_cast<const void*>(kern);
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, Ly::kLds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3((unsigned)(g.BH * (8 / SH::kNcg))), dim3(Ly::kThreads), Ly::kLds,
                       stream, g, stride);
    return hipGetLastError();
}

template <class SH>
hipError_t launch_scan_shape(const GlaLaunch& g, int outk, int stride, hipStream_t stream) {
    if (outk == 1) return launch_scan3<SH, 1>(g, stride, stream);
    if (outk == 2) return launch_scan3<SH, 2>(g, stride, stream);
    return launch_scan3<SH, 0>(g, stride, stream);
}

}  // namespace

size_t gla_fwd_workspace_bytes(int BH, long long L) {
    const long long nch = (L + kC - 1) / kC;
    return (size_t)BH * (size_t)nch * kFBlockBytes;
}

hipError_t launch_gla_fwd(const GlaLaunch& g, hipStream_t stream, int parts) {
    if (g.BH == 0 || g.L == 0) return hipSuccess;
    if (g.d != kD || g.chunk != kC) return hipErrorInvalidValue;
    const long long nch = (g.L + kC - 1) / kC;
    if (g.ws_bytes < gla_fwd_workspace_bytes(g.BH, g.L)) return hipErrorInvalidValue;
    if ((long long)g.BH * nch > 0x7fffffffLL) return hipErrorInvalidValue;
    const int outk = g.o ? (g.out_f32 ? 1 : 2) : 0;
    const int stride = outk ? kFBlockBytes : kFStateBytes;
    if (parts & kGlaPrep) {
        if (outk)
            hipLaunchKernelGGL(gla_prep2_kernel<true>, dim3((unsigned)(g.BH * nch)), dim3(256), 0, stream,
                               g, (int)nch, stride);
        else
            hipLaunchKernelGGL(gla_prep2_kernel<false>, dim3((unsigned)(g.BH * nch)), dim3(256), 0,
                               stream, g, (int)nch, stride);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (parts & kGlaScanNarrow) return launch_scan_shape<NarrowScan>(g, outk, stride, stream);
    if (parts & kGlaScan) return launch_scan_shape<WideScan>(g, outk, stride, stream);
    return hipSuccess;
}

}  // namespace hta
