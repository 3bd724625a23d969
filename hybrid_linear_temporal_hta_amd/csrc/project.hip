// project.hip -- the input side of the GLA branch: per-token projections and
// gates from token features, one bf16 MFMA GEMM with a fused epilogue.
//
// Method: page "Kairos：面向物理 AI 的原生世界模型栈" (yingwang.github.io), section
// 二、方法, second pillar, GLA paragraph: q = W_Q x, k = W_K x, v = W_V x per token,
// beta = sigmoid(W_beta x), and a forget gate alpha in (0, 1) computed from the
// input (read as sigmoid(W_alpha x)). q and k are optionally L2-normalised per
// token and head.
//
// Y = X W with X [M = B*L][Dm] and W [Dm][N], N = 3*H*128 + 2*H (columns q | k |
// v | alpha | beta, head-major within each group). One workgroup computes a
// 128-token x 128-column tile: column tile j < 3H is one head of q, k or v, tile
// 3H holds the 2H gate columns. Workgroups run in groups of four token tiles per
// column tile, so concurrent ones share X and W slices in L2. Four waves in a 2 x 2 arrangement each own a
// 64 x 64 sub-tile (2 x 2 blocks of v_mfma_f32_32x32x16_bf16). X and W tiles of
// 64 along Dm stream into a two-stage LDS ring with direct global->LDS loads:
// A fragments (X rows) are 16-byte reads of chunk-swizzled 128-byte rows, B
// fragments (W columns) transposed reads (ds_read_b64_tr_b16) of row-major
// 256-byte rows. The epilogue parks the fp32 tile in LDS, then each pair of
// threads finishes one token row: the L2 norm of a q / k head, the bf16 store
// into the [B][H][L][d] layout the rest of the library takes, or the sigmoid
// gates into [B][H][L] fp32.
#include <type_traits>

#include "device_common.h"
#include "hta_internal.h"
#include "lds_dma.h"

namespace hta {

namespace {

constexpr int kBM = 128;             // tokens per tile
constexpr int kGroupM = 4;           // token tiles per column tile in the launch order
constexpr int kBN = 128;             // columns per tile (one head of q, k or v)
constexpr int kBK = 64;              // depth per LDS stage
constexpr int kXRow = kBK * 2;       // 128-byte rows of the X tile
constexpr int kWRow = kBN * 2;       // 256-byte rows of the W tile
constexpr int kXTile = kBM * kXRow;  // 16 KiB
constexpr int kWTile = kBK * kWRow;  // 16 KiB
constexpr int kYRow = kBN * 4 + 16;  // fp32 epilogue rows, padded against bank conflicts

// X tile: 16-byte chunk c (of 8) of row r in slot c ^ swzx(r); for the 32 rows a
// fragment read touches, each (row parity, slot) pair is hit by exactly two lanes
// per half-wave, which spreads a read evenly over the 64 banks.
__device__ __forceinline__ int swzx(int r) { return (r >> 1) & 7; }
// W tile (256-byte rows): the same rotation as the attention K/V tiles.
__device__ __forceinline__ int swzw(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

__device__ __forceinline__ float sigmoidf(float z) { return 1.f / (1.f + __expf(-z)); }

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void project_kernel(ProjLaunch p) {
    __shared__ __attribute__((aligned(1024))) char smem[kBM * kYRow];   // >= 2 x (X + W) stages
    static_assert(kBM * kYRow >= 2 * (kXTile + kWTile), "epilogue tile reuses the ring");
    char* const Xs[2] = {smem, smem + kXTile};
    char* const Ws[2] = {smem + 2 * kXTile, smem + 2 * kXTile + kWTile};
    typedef __attribute__((address_space(3))) char lds_char;
    const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_char*)smem;

    const int ntile = 3 * p.H + 1;
    const int nwg = p.nmt * ntile;
    const int wid = xcd_remap(blockIdx.x, nwg);
    // Grouped order: each column tile visits kGroupM token tiles in a row, so the
    // workgroups in flight on one XCD share their X and W slices in its L2 (one
    // token tile with all its column tiles streamed all of W per token tile).
    const int gsz = kGroupM * ntile;
    const int grp = wid / gsz;
    const int first = grp * kGroupM;
    const int gm = min((int)p.nmt - first, kGroupM);
    const int rr = wid - grp * gsz;
    const int mt = first + rr % gm;
    const int nt = rr / gm;
    const long long m0 = (long long)mt * kBM;
    const int n0 = nt * kBN;
    const int nvalid_cols = nt < 3 * p.H ? kBN : 2 * p.H;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int nl = lane & 31, h = lane >> 5;

    // Per-lane offsets: DMA sources / destinations, and fragment reads.
    uint32_t xsrc[4], wsrc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int px = 64 * (4 * wave + i) + lane;              // X: 1024 chunks of 16 B
        const int rx = px >> 3, cx = (px & 7) ^ swzx(rx);
        const long long row = min(m0 + rx, p.M - 1);           // past the end: a valid row
        xsrc[i] = (uint32_t)(((row - m0) * p.Dm + cx * 8) * 2);   // from the tile's first row
        const int pw = 64 * (4 * wave + i) + lane;              // W: 1024 chunks of 16 B
        const int rw = pw >> 4, cw0 = (pw & 15) ^ swzw(rw);
        const int cw = (n0 + 8 * cw0 + 8 <= p.N) ? cw0 : 0;     // gate tile: stay inside W
        wsrc[i] = (uint32_t)(((long long)rw * p.N + 8 * cw) * 2);
    }
    uint32_t xa[2][4];                 // A fragment (row block rb, k-step ks)
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int r = 64 * wm + 32 * rb + nl;
            xa[rb][ks] = r * kXRow + 16 * ((2 * ks + h) ^ swzx(r));
        }
    // B fragment (column block cb) by two transposed reads per k-step. Within a
    // 16-lane group g, lane 4j + a addresses row 8(g/2) + j (then + 4), columns
    // 16(g%2) + 4a .. +3; the read hands lane 4a + b column b of those four rows,
    // so lane l ends up with rows 8(l/32) .. +7 of column l%32: the natural k
    // order of the MFMA B operand, matching the A fragments' 16-byte reads.
    uint32_t wb[2][2];
    {
        const int g = lane >> 4, sl = lane & 15, jr = sl >> 2, ac = sl & 3;
        const int r0 = 8 * (g >> 1) + jr, r1 = r0 + 4;
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
            const int col = 64 * wn + 32 * cb + 16 * (g & 1) + 4 * ac;
            wb[cb][0] = r0 * kWRow + 16 * ((col >> 3) ^ swzw(r0)) + 8 * ((col >> 2) & 1);
            wb[cb][1] = r1 * kWRow + 16 * ((col >> 3) ^ swzw(r1)) + 8 * ((col >> 2) & 1);
        }
    }

    const bf16* xbase = static_cast<const bf16*>(p.x) + m0 * p.Dm;
    const bf16* wbase = static_cast<const bf16*>(p.w) + n0;
    auto issue = [&](int kt, int st) {
        const bf16* xs = xbase + (long long)kt * kBK;
        const bf16* ws = wbase + (long long)kt * kBK * p.N;
        const uint32_t lx = lds0 + st * kXTile, lw = lds0 + 2 * kXTile + st * kWTile;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t off = 1024u * (4 * wave + i);
            dma16(xsrc[i], xs, lx + off);
            dma16(wsrc[i], ws, lw + off);
        }
    };

    f32x16 acc[2][2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[rb][cb][i] = 0.f;

    const int nk = p.Dm / kBK;
    issue(0, 0);
    auto step = [&](int kt, auto stage_tag) {
        constexpr int ST = decltype(stage_tag)::value;
        wait_vmcnt<0>();   // this stage's loads have landed ...
        __syncthreads();     // ... for every wave; the other stage was read by all
        if (kt + 1 < nk) issue(kt + 1, ST ^ 1);
        typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            bf16x8 a[2], b[2];
#pragma unroll
            for (int rb = 0; rb < 2; ++rb)
                a[rb] = *reinterpret_cast<const bf16x8*>(Xs[ST] + xa[rb][ks]);
            const char* wk = Ws[ST] + 16 * ks * kWRow;
#pragma unroll
            for (int cb = 0; cb < 2; ++cb) {
                const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(wk + wb[cb][0]));
                const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(wk + wb[cb][1]));
                b[cb] = cat(lo, hi);
            }
#pragma unroll
            for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                for (int cb = 0; cb < 2; ++cb) acc[rb][cb] = mfma32(a[rb], b[cb], acc[rb][cb]);
        }
    };
    for (int kt = 0; kt < nk; kt += 2) {
        step(kt, std::integral_constant<int, 0>{});
        if (kt + 1 < nk) step(kt + 1, std::integral_constant<int, 1>{});
    }

    // Epilogue: the fp32 tile into LDS (element i of block (rb, cb) is row
    // 8(i/4) + 4h + i%4, column nl of that 32 x 32 block).
    __syncthreads();
    float* Ys = reinterpret_cast<float*>(smem);
    constexpr int kYf = kYRow / 4;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int r = 64 * wm + 32 * rb + 8 * (i >> 2) + 4 * h + (i & 3);
                const int c = 64 * wn + 32 * cb + nl;
                Ys[r * kYf + c] = acc[rb][cb][i];
            }
    __syncthreads();

    const int t = threadIdx.x;
    if (nt < 3 * p.H) {
        // Two threads per token row, 64 columns each.
        const int r = t >> 1, half = t & 1;
        const long long m = m0 + r;
        const int grp = nt / p.H, head = nt - grp * p.H;
        const bool norm = (grp == 0 && (p.flags & 1)) || (grp == 1 && (p.flags & 2));
        const float* yr = Ys + r * kYf + 64 * half;
        f32x4 y[16];
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            y[i] = *reinterpret_cast<const f32x4*>(yr + 4 * i);
#pragma unroll
            for (int j = 0; j < 4; ++j) ss += y[i][j] * y[i][j];
        }
        ss += __shfl_xor(ss, 1, 64);
        const float sc = norm ? (ss > 0.f ? 1.f / sqrtf(ss) : 0.f) : 1.f;
        if (m < p.M) {
            const long long b = m / p.L, tok = m - b * p.L;
            bf16* out = static_cast<bf16*>(grp == 0 ? p.q : grp == 1 ? p.k : p.v);
            bf16* dst = out + (((b * p.H + head) * p.L + tok) * kBN) + 64 * half;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                bf16x8 o;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    o[j] = f2bf(y[2 * i][j] * sc);
                    o[4 + j] = f2bf(y[2 * i + 1][j] * sc);
                }
                *reinterpret_cast<bf16x8*>(dst + 8 * i) = o;
            }
        }
    } else {
        // Gate tile: column c < H is alpha of head c, H <= c < 2H beta of head c - H.
        for (int e = t; e < kBM * nvalid_cols; e += 256) {
            const int r = e % kBM, c = e / kBM;
            const long long m = m0 + r;
            if (m >= p.M) continue;
            const long long b = m / p.L, tok = m - b * p.L;
            const int head = c < p.H ? c : c - p.H;
            float* out = c < p.H ? p.alpha : p.beta;
            out[(b * p.H + head) * p.L + tok] = sigmoidf(Ys[r * kYf + c]);
        }
    }
}

}  // namespace

hipError_t launch_project(const ProjLaunch& p, hipStream_t stream) {
    if (p.M == 0) return hipSuccess;
    const long long nwg = p.nmt * (3LL * p.H + 1);
    if (nwg > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL(project_kernel, dim3((unsigned)nwg), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace hta
