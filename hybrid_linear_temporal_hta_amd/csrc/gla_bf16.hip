// gla_bf16.hip -- the chunked gated-delta GLA forward that the GLA backward
// re-runs (gfx950, bf16 in, fp32 state): besides the final state it saves, per
// chunk, the state entering it (M0) and U, in fp16, for the reverse scan and the
// chunk gradients. (The inference forward is gla_fwd.hip.)
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
// Precision: inputs are bf16 and every accumulation is fp32; the operands the
// kernels build themselves (K and Q re-expressed in fp16 -- exact --, T, Pm,
// the state copy fed to K M0 / Q M0, X, U) are fp16, whose 11-bit significand
// keeps the chunk algebra about 8x closer to exact than bf16 operands would.
// fp16 bounds their range: the backward hands the scan V and the initial state
// multiplied by a power of two sigma_v (GlaLaunch::vscale) that maps their largest
// magnitude into [1, 2), so the fp16 operands stay in range for any finite v and
// state as long as the update does not grow the state beyond ~3e4 times that
// maximum (with unit-norm keys and alpha < 1 the state stays within
// max|v| sqrt(d) / sqrt(1 - alpha^2)); saved M0 and U then carry the same factor.
//
// Two kernels:
//   prep (one workgroup per chunk, all chunks in parallel): g, A and Pm from
//     K K^T and Q K^T on v_mfma_f32_32x32x16_bf16, T in fp32 by 16x16 blocks
//     (diagonal blocks by forward substitution, the blocks below them by fp32
//     MFMA products), and the chunk's operand block -- K, Q (fp16), T, Pm
//     (fp16), e^{g}, e^{g_C - g}, beta, e^{gp} (fp32) -- written contiguously in
//     exactly the LDS layout the scan consumes (swizzles included).
//
// The printed form of the update (GlaLaunch::form = 1: the erase term uses the
// state before the forget gate, S_t = alpha S - beta (S k) k^T + beta v k^T)
// differs only where the chunk predicts values from the state: A and the K M0
// term of X take e^{g_{i-1}} (exclusive cumulative sum, "gp") instead of e^{g_i}.
// Pm, the output and the state update are the same.
//   scan (one workgroup per (batch, head, 64 value columns), chunks in order):
//     eight waves in two roles over the same 16-column groups. State waves hold
//     their 16 value columns of the fp32 state as eight 16x16 MFMA accumulator
//     tiles and run the recurrence (K M0, T X, K^T U on v_mfma_f32_16x16x32_f16;
//     the B operands that are previous results -- M0, X, U -- come straight
//     from accumulator registers, token order permuted identically in A and B;
//     K^T fragments are transposed LDS reads of row-major K). Output waves
//     stream the next chunk's operand block and value tile into the other half
//     of a two-stage LDS ring with direct global->LDS loads, and form and store
//     the output from the M0 and U the state waves hand over in LDS.
#include <type_traits>

#include "device_common.h"
#include "gla_tiles.h"
#include "hta_internal.h"

namespace hta {

namespace {

using namespace glat;

// ------------------------------------------------------------------ prep

constexpr int kKsP = kD + 8;      // padded K / Q row (bf16)
constexpr int kAsP = 68;          // padded A / T row (fp32)
static_assert(kC * kKsP * 2 == kC * kAsP * 4, "Q staging shares the A buffer; T the K buffer");
static_assert(kC * kKsP * 2 >= 64 * 128, "Pm and T staging fit in a buffer");

// One workgroup per chunk. Phases, separated by barriers:
//   1. loads: alpha, beta (wave 0), K and Q rows; K and Q kept in LDS as bf16 and
//      written to the block as fp16; the decay prefix sums (wave 0);
//   2. K K^T and Q K^T on MFMA, one 32x32 block per wave;
//   3. A into LDS (the Q buffer), Pm into LDS staging in the block layout;
//   4. Pm copied out with 16-byte stores; T = (I + A)^-1 in fp32 by 16x16 blocks
//      (the K buffer): each wave inverts one diagonal block by forward
//      substitution, then the blocks below the diagonal follow in three levels of
//      products, T_ik = -T_ii sum_{k <= j < i} A_ij T_jk (from (I + A) T = I);
//      T is staged in fp16 in the block layout (the A buffer) and copied out last.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4)))
void gla_prep_bf16_kernel(GlaLaunch g, int nch) {
    __shared__ __attribute__((aligned(16))) bf16 Ks[kC * kKsP];   // K; then Pm staging, then T (fp32)
    __shared__ __attribute__((aligned(16))) float As[kC * kAsP];  // Q (bf16); then A; then T staging[i][(j&3)*16 + (j>>2)]
    __shared__ float gs[kC];
    __shared__ float gps[kC];   // decay exponent of the erase path (see kOffX)
    __shared__ float bs[kC];
    bf16* Qs = reinterpret_cast<bf16*>(As);
    char* stP = reinterpret_cast<char*>(Ks);          // Pm, 8 KiB, block layout

    const int cid = blockIdx.x;
    const int bh = cid / nch, c = cid - bh * nch;
    const long long t0 = (long long)c * kC;
    const int n = (int)min((long long)kC, g.L - t0);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const bf16* kp = static_cast<const bf16*>(g.k) + ((long long)bh * g.L + t0) * kD;
    const bf16* qp = static_cast<const bf16*>(g.q) + ((long long)bh * g.L + t0) * kD;
    char* blk = static_cast<char*>(g.ws) + (size_t)cid * kChunkBytes;

    float alpha_t = 1.f, beta_t = 0.f;
    if (wave == 0 && lane < n) {
        alpha_t = g.alpha[(long long)bh * g.L + t0 + lane];
        beta_t = g.beta[(long long)bh * g.L + t0 + lane];
    }
    u32x4 kv[4], qv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int ci = tid + 256 * r, row = ci >> 4, cc = ci & 15;
        kv[r] = u32x4{0u, 0u, 0u, 0u};
        qv[r] = u32x4{0u, 0u, 0u, 0u};
        if (row < n) {
            kv[r] = *reinterpret_cast<const u32x4*>(kp + (long long)row * kD + 8 * cc);
            qv[r] = *reinterpret_cast<const u32x4*>(qp + (long long)row * kD + 8 * cc);
        }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int ci = tid + 256 * r, row = ci >> 4, cc = ci & 15;
        *reinterpret_cast<u32x4*>(Ks + row * kKsP + 8 * cc) = kv[r];
        *reinterpret_cast<u32x4*>(Qs + row * kKsP + 8 * cc) = qv[r];
        *reinterpret_cast<u32x4*>(blk + kOffK + offK(row, 8 * cc)) = bf16x8_to_f16x8(kv[r]);
        *reinterpret_cast<u32x4*>(blk + kOffQ + offK(row, 8 * cc)) = bf16x8_to_f16x8(qv[r]);
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
        const float gC = __shfl(la, 63, 64);
        const float prev = __shfl_up(la, 1, 64);
        const float gp = g.form ? (lane == 0 ? 0.f : prev) : la;
        gs[lane] = la;
        gps[lane] = gp;
        bs[lane] = beta_t;
        reinterpret_cast<float*>(blk + kOffE)[lane] = __expf(la);
        reinterpret_cast<float*>(blk + kOffD)[lane] = __expf(gC - la);
        reinterpret_cast<float*>(blk + kOffB)[lane] = beta_t;
        reinterpret_cast<float*>(blk + kOffX)[lane] = __expf(gp);
    }
    __syncthreads();

    // K K^T and Q K^T, one 32x32 block per wave.
    const int mb = wave >> 1, nb = wave & 1;
    const int nn = lane & 31, h = lane >> 5;
    f32x16 kk, qk;
#pragma unroll
    for (int i = 0; i < 16; ++i) { kk[i] = 0.f; qk[i] = 0.f; }
    if (mb >= nb) {
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            const bf16x8 ka = *reinterpret_cast<const bf16x8*>(Ks + (mb * 32 + nn) * kKsP + 16 * ks + 8 * h);
            const bf16x8 kb = *reinterpret_cast<const bf16x8*>(Ks + (nb * 32 + nn) * kKsP + 16 * ks + 8 * h);
            const bf16x8 qa = *reinterpret_cast<const bf16x8*>(Qs + (mb * 32 + nn) * kKsP + 16 * ks + 8 * h);
            kk = mfma32(ka, kb, kk);
            qk = mfma32(qa, kb, qk);
        }
    }
    __syncthreads();   // K and Q read by every wave: their buffers are reused below
    {
        const int j = nb * 32 + nn;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int i = mb * 32 + 8 * (e >> 2) + 4 * h + (e & 3);
            const float dec = (j <= i) ? __expf(gs[i] - gs[j]) : 0.f;
            const float deca = (j < i) ? __expf(gps[i] - gs[j]) : 0.f;
            As[i * kAsP + j] = (j < i) ? bs[i] * deca * kk[e] : 0.f;
            *reinterpret_cast<f16*>(stP + offT(i, j)) = (f16)((j <= i) ? dec * qk[e] : 0.f);
        }
    }
    __syncthreads();

    // Pm to the block, 16 bytes per thread and step
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int q = tid + 256 * r;
        *reinterpret_cast<u32x4*>(blk + kOffP + 16 * q) = *reinterpret_cast<const u32x4*>(stP + 16 * q);
    }

    // Diagonal block kb = wave of T by forward substitution: lane (column c, sub)
    // keeps x_r for the block's rows r = 4 m + sub (entries not yet solved are 0,
    // and so is A on and above the diagonal, so every product term is safe).
    float* Ts = reinterpret_cast<float*>(Ks);   // T, fp32 [64][kAsP]
    {
        const int kb = wave, c = lane >> 2, sub = lane & 3;
        const float* Ab = As + 16 * kb * kAsP + 16 * kb;
        float x[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float* ar = Ab + i * kAsP + sub;
            float part = (ar[0] * x[0] + ar[4] * x[1]) + (ar[8] * x[2] + ar[12] * x[3]);
            part += quad_xor1(part);   // sum over the quad's four lanes, in registers
            part += quad_xor2(part);
            const float xi = (i == c ? 1.f : 0.f) - part;
            if ((i & 3) == sub) x[i >> 2] = xi;
        }
        __syncthreads();   // the Pm staging (same buffer) has been copied out
#pragma unroll
        for (int m = 0; m < 4; ++m) Ts[(16 * kb + 4 * m + sub) * kAsP + 16 * kb + c] = x[m];
    }
    __syncthreads();
    // Blocks (k + d, k) at level d, wave k: S = sum_j A_ij T_jk, then T_ik = -T_ii S
    // (S staged in the block's own slot: each wave reads it back before overwriting).
    {
        const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
        const int n = lane & 15, g = lane >> 4;
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
                for (int r = 0; r < 4; ++r) Tik[(4 * g + r) * kAsP + n] = sacc[r];
                const f32x4 t = mm16f(Ts + 16 * i * kAsP + 16 * i, kAsP, Tik, kAsP, zero4, lane);
#pragma unroll
                for (int r = 0; r < 4; ++r) Tik[(4 * g + r) * kAsP + n] = -t[r];
            }
            __syncthreads();
        }
    }
    // T (lower triangular, unit diagonal) in fp16, staged in the block layout in the A buffer
    char* stT = reinterpret_cast<char*>(As);
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int q = tid + 256 * r, i = q >> 3, j0 = (q & 7) * 8;
        const float* tr = Ts + i * kAsP + j0;
        f16x8 h8;
#pragma unroll
        for (int u = 0; u < 8; ++u) h8[u] = (f16)((j0 + u <= i) ? tr[u] : 0.f);
        *reinterpret_cast<f16x8*>(stT + offT(i, j0)) = h8;
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int q = tid + 256 * r;
        *reinterpret_cast<u32x4*>(blk + kOffT + 16 * q) = *reinterpret_cast<const u32x4*>(stT + 16 * q);
    }
}

// ------------------------------------------------------------------ scan

// LDS of the scan: two operand stages, then the hand-over from the state waves
// to the output waves: M0 (the state entering the chunk) and U, both already
// rounded to the fp16 B fragments the products consume. Fragment k of lane l of
// column group w sits at ((w * nfrag + k) * 64 + l) * 16: consecutive lanes,
// consecutive 16-byte slots.
constexpr int kXchM = 2 * kStageBytes;
constexpr int kXchU = kXchM + 4 * 4 * 64 * 16;
constexpr int kScanLds = kXchU + 4 * 2 * 64 * 16;
// With the states saved for a backward pass: per output wave, a column-major
// staging of its 16 columns (kSaveCol bytes per column: up to 128 rows + padding
// that spreads the banks) for the transposed copy-out.
constexpr int kSaveCol = 288;
constexpr int kSaveSt = kScanLds;
constexpr int kScanLdsSave = kSaveSt + 4 * 16 * kSaveCol;
static_assert(kScanLdsSave <= 160 * 1024, "scan LDS exceeds one CU");

// Copy a wave's NF fp16 B fragments of its 16 columns -- fragment k holds rows
// 32k + 4G + i and 32k + 16 + 4G + i (i < 4) of column m -- to the row-major
// [rows][kD] tensor at dst (which points at the wave's first column): staged
// column by column in LDS, read back by transposed reads as rows of 8 columns,
// and stored 16 bytes per lane.
template <int NF>
__device__ __forceinline__ void save_rows(char* st, const f16x8 (&fr)[NF], f16* dst, int lane) {
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    const int m = lane & 15, G = lane >> 4;
#pragma unroll
    for (int k = 0; k < NF; ++k) {
        *reinterpret_cast<f16x4*>(st + m * kSaveCol + (32 * k + 4 * G) * 2) =
            f16x4{fr[k][0], fr[k][1], fr[k][2], fr[k][3]};
        *reinterpret_cast<f16x4*>(st + m * kSaveCol + (32 * k + 16 + 4 * G) * 2) =
            f16x4{fr[k][4], fr[k][5], fr[k][6], fr[k][7]};
    }
    // block q: rows 16 (q >> 1) .. +15, columns 8 (q & 1) .. +7. In a transposed
    // read, source lane 4j + a addresses staged column c + j at rows r0 + 4a .. +3,
    // and lane 4a + b receives row r0 + 4a + b of columns c .. c + 3.
    const int j = m >> 2, a = m & 3;
#pragma unroll
    for (int t = 0; t < NF; ++t) {
        const int q = G + 4 * t, r0 = 16 * (q >> 1), c0 = 8 * (q & 1);
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4*)(st + (c0 + j) * kSaveCol + (r0 + 4 * a) * 2));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4*)(st + (c0 + 4 + j) * kSaveCol + (r0 + 4 * a) * 2));
        *reinterpret_cast<f16x8*>(dst + (r0 + m) * kD + c0) =
            cat(__builtin_bit_cast(f16x4, lo), __builtin_bit_cast(f16x4, hi));
    }
}

// Enqueue chunk c's operand block and 64-column V tile into an LDS stage; ow is
// the issuing wave among the four output waves.
__device__ __forceinline__ void issue_chunk(char* stage, const GlaLaunch& g, int bh, int tile,
                                            long long c, long long nch, int ow, int lane) {
    const char* blk = static_cast<const char*>(g.ws) + (size_t)((long long)bh * nch + c) * kChunkBytes;
#pragma unroll
    for (int i = 0; i < 12; ++i) {
        const int q = 12 * ow + i;
        dma16p(blk + 1024 * q + 16 * lane, stage + 1024 * q);
    }
    if (ow == 0 && lane < kTailChunks) dma16p(blk + kBlockMain + 16 * lane, stage + kBlockMain);
    const long long t0 = c * kC;
    const int n = (int)min((long long)kC, g.L - t0);
    const bf16* vb = static_cast<const bf16*>(g.v) + ((long long)bh * g.L + t0) * kD + tile * 64;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int p = 64 * (2 * ow + i) + lane;
        const int tok = p >> 3;
        const int cc = (p & 7) ^ swzv(tok);
        dma16p(vb + (long long)min(tok, n - 1) * kD + 8 * cc, stage + kOffV + 1024 * (2 * ow + i));
    }
}

// One workgroup per (batch, head, 64 value columns), eight waves in two roles
// that share the column group cg = wave & 3 (16 columns each):
//   state waves (0..3) carry the recurrence: K M0, X, U = T X and the update of
//     M; they publish M0 and U to LDS and never touch global memory inside the
//     loop;
//   output waves (4..7) issue the next chunk's DMA, store the saved M0 / U when
//     asked, and form the output O = diag(e^g) Q M0 + Pm U and store it, 16 bytes
//     per lane.
// Two barriers per chunk: B1 (chunk c staged, M0 published) and B2 (U published).
// The arithmetic and its rounding are those of a single wave doing both.
template <bool OUT_F32>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gla_scan_bf16_kernel(GlaLaunch g) {
    extern __shared__ __attribute__((aligned(1024))) char smem[];

    const int BH = g.BH;
    const int b = blockIdx.x;
    int bh, tile;
    if ((BH & 7) == 0) { bh = (b & 7) + 8 * (b >> 4); tile = (b >> 3) & 1; }   // both tiles of a head on one XCD
    else { bh = b >> 1; tile = b & 1; }
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool state_wave = wave < 4;
    const int cg = wave & 3;
    const int m = lane & 15, G = lane >> 4;
    const int col = tile * 64 + cg * 16 + m;
    const long long nch = (g.L + kC - 1) / kC;
    f16x8* xm = reinterpret_cast<f16x8*>(smem + kXchM) + cg * 4 * 64 + lane;   // + 64 k
    f16x8* xu = reinterpret_cast<f16x8*>(smem + kXchU) + cg * 2 * 64 + lane;
    float* st = g.state + (long long)bh * kD * kD;
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};

    if (state_wave) {
        const float sv = g.vscale ? sigma_of(*g.vscale) : 1.f;
        f32x4 Mr[8];                                   // sv M[16kb + 4G + i][col]
#pragma unroll
        for (int kb = 0; kb < 8; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i) Mr[kb][i] = st[(16 * kb + 4 * G + i) * kD + col] * sv;
        f16x8 bM[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            bM[ks] = bfrag(Mr[2 * ks], Mr[2 * ks + 1]);
            xm[64 * ks] = bM[ks];
        }
        for (long long c = 0; c < nch; ++c) {
            __syncthreads();   // B1: chunk c staged; the output waves have M0
            const char* S = smem + (c & 1) * kStageBytes;
            const float* esm = reinterpret_cast<const float*>(S + kOffE);
            const float* dsm = reinterpret_cast<const float*>(S + kOffD);
            const float* bsm = reinterpret_cast<const float*>(S + kOffB);
            const float* xsm = reinterpret_cast<const float*>(S + kOffX);
            // K M0
            f16x8 kf[4][4];
#pragma unroll
            for (int rb = 0; rb < 4; ++rb)
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) kf[rb][ks] = afragK(S + kOffK, 16 * rb + m, ks, G);
            f32x4 KM[4];
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) {
                KM[rb] = zero4;
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) KM[rb] = mfma16h(kf[rb][ks], bM[ks], KM[rb]);
            }
            f16x8 tf[4][2];
#pragma unroll
            for (int rb = 0; rb < 4; ++rb)
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
                    if (kt == 0 || rb >= 2) tf[rb][kt] = afragT(S + kOffT, 16 * rb + m, kt, G);
            // Per-token factors of this lane's rows 16rb + 4G + i, four at a time.
            f32x4 d4[4], b4[4], x4[4];
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) {
                x4[rb] = *reinterpret_cast<const f32x4*>(xsm + 16 * rb + 4 * G);
                d4[rb] = *reinterpret_cast<const f32x4*>(dsm + 16 * rb + 4 * G);
                b4[rb] = *reinterpret_cast<const f32x4*>(bsm + 16 * rb + 4 * G);
            }
            // V[16rb + 4G + i][col], i = 0..3, by one transposed read per row block:
            // source lane 4j + a addresses token 16rb + 4G + j, columns 16cg + 4a .. +3.
            bf16x4 v4[4];
            {
                typedef short s16x4 __attribute__((ext_vector_type(4)));
                typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
                const int j = m >> 2, a = m & 3;
                const int vc = 16 * cg + 4 * a;
#pragma unroll
                for (int rb = 0; rb < 4; ++rb) {
                    const int t = 16 * rb + 4 * G + j;
                    const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(
                        S + kOffV + t * 128 + 16 * ((vc >> 3) ^ swzv(t)) + 2 * (vc & 7)));
                    v4[rb] = __builtin_bit_cast(bf16x4, r);
                }
            }
            // X = diag(beta) (V - diag(e^gp) K M0)
            f32x4 X[4];
#pragma unroll
            for (int rb = 0; rb < 4; ++rb)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    X[rb][i] = b4[rb][i] * (bf2f(v4[rb][i]) * sv - x4[rb][i] * KM[rb][i]);
            const f16x8 xb[2] = {bfrag(X[0], X[1]), bfrag(X[2], X[3])};
            // U = T X (T lower triangular: row blocks 0,1 only see k-step 0)
            f32x4 U[4];
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) {
                U[rb] = mfma16h(tf[rb][0], xb[0], zero4);
                if (rb >= 2) U[rb] = mfma16h(tf[rb][1], xb[1], U[rb]);
            }
            xu[0] = bfrag(U[0], U[1]);
            xu[64] = bfrag(U[2], U[3]);
            f32x4 Us[4];
#pragma unroll
            for (int rb = 0; rb < 4; ++rb)
#pragma unroll
                for (int i = 0; i < 4; ++i) Us[rb][i] = U[rb][i] * d4[rb][i];
            const f16x8 usb[2] = {bfrag(Us[0], Us[1]), bfrag(Us[2], Us[3])};
            const float egC = esm[kC - 1];
            __syncthreads();   // B2: U published; the output waves are done with M0
            // M = e^{g_C} M0 + K^T diag(e^{g_C - g}) U
#pragma unroll
            for (int kb = 0; kb < 8; ++kb) {
                const f16x8 k0 = afragKt(S + kOffK, kb, 0, lane);
                const f16x8 k1 = afragKt(S + kOffK, kb, 1, lane);
#pragma unroll
                for (int i = 0; i < 4; ++i) Mr[kb][i] *= egC;
                Mr[kb] = mfma16h(k0, usb[0], Mr[kb]);
                Mr[kb] = mfma16h(k1, usb[1], Mr[kb]);
            }
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                bM[ks] = bfrag(Mr[2 * ks], Mr[2 * ks + 1]);
                xm[64 * ks] = bM[ks];
            }
        }
#pragma unroll
        for (int kb = 0; kb < 8; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i) st[(16 * kb + 4 * G + i) * kD + col] = Mr[kb][i] / sv;
    } else {
        const float scale = g.scale / (g.vscale ? sigma_of(*g.vscale) : 1.f);
        issue_chunk(smem, g, bh, tile, 0, nch, cg, lane);
        for (long long c = 0; c < nch; ++c) {
            wait_vmcnt<0>();     // this wave's part of chunk c has landed
            __syncthreads();   // B1
            if (c + 1 < nch) issue_chunk(smem + ((c + 1) & 1) * kStageBytes, g, bh, tile, c + 1, nch, cg, lane);
            const char* S = smem + (c & 1) * kStageBytes;
            f16x8 bM[4];
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) bM[ks] = xm[64 * ks];
            if (g.save_m)   // the state entering this chunk, for a backward pass
                save_rows<4>(smem + kSaveSt + cg * 16 * kSaveCol, bM,
                             static_cast<f16*>(g.save_m) + ((long long)bh * nch + c) * kD * kD +
                                 tile * 64 + cg * 16,
                             lane);
            // The output is formed transposed, O^T = M0^T Q^T + U^T Pm^T: an A fragment
            // and a B fragment of the 16x16x32 product have the same lane layout, so the
            // same registers serve with the operands swapped, and lane (m, G) ends up
            // holding O[16 rb + m][16 cg + 4G + i], four adjacent columns of one token.
            f32x4 QM[4];
            if (g.o) {
#pragma unroll
                for (int rb = 0; rb < 4; ++rb) {
                    QM[rb] = zero4;
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks)
                        QM[rb] = mfma16h(bM[ks], afragK(S + kOffQ, 16 * rb + m, ks, G), QM[rb]);
                }
            }
            __syncthreads();   // B2
            const f16x8 ub[2] = {xu[0], xu[64]};
            if (g.save_u)
                save_rows<2>(smem + kSaveSt + cg * 16 * kSaveCol, ub,
                             static_cast<f16*>(g.save_u) + ((long long)bh * nch + c) * kC * kD +
                                 tile * 64 + cg * 16,
                             lane);
            if (g.o) {
                const float* esm = reinterpret_cast<const float*>(S + kOffE);
                const long long t0 = c * kC;
                const int c0 = tile * 64 + cg * 16 + 4 * G;
#pragma unroll
                for (int rb = 0; rb < 4; ++rb) {
                    f32x4 PU = mfma16h(ub[0], afragT(S + kOffP, 16 * rb + m, 0, G), zero4);
                    if (rb >= 2) PU = mfma16h(ub[1], afragT(S + kOffP, 16 * rb + m, 1, G), PU);
                    const int tok = 16 * rb + m;
                    const float e = esm[tok];
                    f32x4 ov;
#pragma unroll
                    for (int i = 0; i < 4; ++i) ov[i] = scale * (e * QM[rb][i] + PU[i]);
                    if (t0 + tok < g.L) {
                        const long long off = ((long long)bh * g.L + t0 + tok) * kD + c0;
                        if (OUT_F32) {
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
        wait_vmcnt<0>();
    }
}

}  // namespace

size_t gla_bf16_chunk_bytes() { return kChunkBytes; }

size_t gla_bf16_workspace_bytes(int BH, long long L, int chunk) {
    (void)chunk;
    const long long nch = (L + kC - 1) / kC;
    return (size_t)BH * (size_t)nch * kChunkBytes;
}

hipError_t launch_gla_bf16(const GlaLaunch& g, hipStream_t stream, int parts) {
    if (g.BH == 0 || g.L == 0) return hipSuccess;
    if (g.d != kD || g.chunk != kC) return hipErrorInvalidValue;
    const long long nch = (g.L + kC - 1) / kC;
    if (g.ws_bytes < gla_bf16_workspace_bytes(g.BH, g.L, g.chunk)) return hipErrorInvalidValue;
    if ((long long)g.BH * nch > 0x7fffffffLL) return hipErrorInvalidValue;
    hipError_t e;
    if (parts & kGlaPrep) {
        hipLaunchKernelGGL(gla_prep_bf16_kernel, dim3((unsigned)(g.BH * nch)), dim3(256), 0, stream,
                           g, (int)nch);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (!(parts & kGlaScan)) return hipSuccess;
    // > 64 KiB: raise the launch limit (current device)
    const size_t smem = (g.save_m || g.save_u) ? kScanLdsSave : kScanLds;
    const void* fn = g.out_f32 ? reinterpret_cast<const void*>(gla_scan_bf16_kernel<true>)
                               : reinterpret_cast<const void*>(gla_scan_bf16_kernel<false>);
    e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kScanLdsSave);
    if (e != hipSuccess) return e;
    if (g.out_f32)
        hipLaunchKernelGGL(gla_scan_bf16_kernel<true>, dim3((unsigned)(g.BH * 2)), dim3(512), smem, stream, g);
    else
        hipLaunchKernelGGL(gla_scan_bf16_kernel<false>, dim3((unsigned)(g.BH * 2)), dim3(512), smem, stream, g);
    return hipGetLastError();
}

}  // namespace hta
