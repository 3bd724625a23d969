/*
 * oracle.c -- plain, slow, obviously-correct fp64 CPU oracle for Hybrid Linear
 * Temporal Attention (HLTA): sliding-window attention (SWA), dilated
 * sliding-window attention (DSWA) and gated linear attention with the gated
 * delta update (GLA).
 *
 * TEST INFRASTRUCTURE. Only the test-suite, the smoke entry point and the
 * benchmark's CPU-baseline leg may load this library. It shares no source,
 * header, table or helper with the HIP library; neither includes the other.
 *
 * Sources (web pages describing the Kairos world model):
 *   [P1] "Kairos：面向物理 AI 的原生世界模型栈" (yingwang.github.io, paper-reads),
 *        section 二、方法 (Method), second pillar (unified architecture):
 *        the SWA paragraph, the DSWA paragraph (dilation d, re-layout
 *        (B, F*L, D) -> (B*d, F/d*L, D)), the GLA paragraph with its update
 *        equations, and the three-branch figure that merges into one mixed
 *        temporal representation.
 *   [P2] "Kairosとは？物理AIの世界モデル基盤…" (ai-papers.net), section
 *        3層ハイブリッド時間アーキテクチャ (three-layer hybrid temporal architecture).
 *
 * Readings taken where the pages leave a step open (each is also listed in
 * the design notes of the repository):
 *   - Tokens are frame-major: token t belongs to frame floor(t / P).
 *   - SWA: a query in frame f attends, with full softmax attention, to every
 *     key in frames f-W+1 .. f (clipped at 0), i.e. the window counts the
 *     current frame, is block-causal across frames and full inside a frame.
 *   - DSWA: the same window size counted in taps; tap j is frame f - j*dil;
 *     taps before frame 0 are absent (not zero-padded keys).
 *   - Softmax logits are scale * q.k with scale = 1/sqrt(dk) unless given.
 *   - GLA follows the GatedDeltaNet form that [P1] names as its basis:
 *       v_old = S_{t-1} k_t
 *       S_t   = alpha_t (S_{t-1} - beta_t v_old k_t^T) + beta_t v_t k_t^T
 *       o_t   = scale * S_t q_t          (post-update state, scale = 1)
 *     S is dv x dk. The carried state crosses the boundary as S^T, laid out
 *     [dk][dv]. The literal three-line form printed in [P1] (forget gate not
 *     applied to the erase term) is kept as oracle_gla_literal.
 *   - Hybrid output: unweighted sum of the three branch outputs.
 *
 * Layout of every sequence tensor: [B][H][L][d] row-major, L = T * P.
 * All arithmetic is fp64; callers pass values already rounded to the storage
 * dtype of the tested path, widened exactly to double.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_OK 0
#define ORC_EARG (-1)
#define ORC_ENOMEM (-2)

/*
 * Softmax attention of one query row over every key of the listed frames
 * ("standard attention restricted to a window", [P1] SWA paragraph).
 * kbh / vbh point at the first key / value row of one (batch, head) slice.
 */
static int attend_frames(const double *qrow, const double *kbh, const double *vbh,
                         int P, int dk, int dv, const int *frames, int nf,
                         double scale, double *out)
{
    long nkeys = (long)nf * P;
    double *z = (double *)malloc(sizeof(double) * (size_t)(nkeys > 0 ? nkeys : 1));
    if (!z) return ORC_ENOMEM;
    double m = -INFINITY;
    long n = 0;
    for (int a = 0; a < nf; ++a) {
        for (int p = 0; p < P; ++p) {
            const double *kr = kbh + ((long)frames[a] * P + p) * dk;
            double s = 0.0;
            for (int i = 0; i < dk; ++i) s += qrow[i] * kr[i];
            s *= scale;
            z[n++] = s;
            if (s > m) m = s;
        }
    }
    for (int j = 0; j < dv; ++j) out[j] = 0.0;
    double den = 0.0;
    n = 0;
    for (int a = 0; a < nf; ++a) {
        for (int p = 0; p < P; ++p) {
            const double *vr = vbh + ((long)frames[a] * P + p) * dv;
            double w = exp(z[n++] - m);
            den += w;
            for (int j = 0; j < dv; ++j) out[j] += w * vr[j];
        }
    }
    for (int j = 0; j < dv; ++j) out[j] /= den;
    free(z);
    return ORC_OK;
}

/* Key frames of SWA for query frame f: f, f-1, ..., f-W+1, those >= 0. */
static int swa_frames(int f, int window, int *frames)
{
    int n = 0;
    for (int j = 0; j < window; ++j)
        if (f - j >= 0) frames[n++] = f - j;
    return n;
}

/* Key frames of DSWA for query frame f: f - j*dil for j < taps, those >= 0. */
static int dswa_frames(int f, int taps, int dil, int *frames)
{
    int n = 0;
    for (int j = 0; j < taps; ++j)
        if (f - j * dil >= 0) frames[n++] = f - j * dil;
    return n;
}

/*
 * Windowed attention for an explicit list of query rows.
 * rows[r] is the flat token index bh*L + t the query sits at (it fixes the key
 * window); qrows[r] is that query's vector ([n_rows][dk]). out is [n_rows][dv].
 * kind 0 = SWA (a = window), kind 1 = DSWA (a = taps, b = dilation).
 */
static int window_rows(int kind, int B, int H, int T, int P, int dk, int dv,
                       const double *qrows, const double *k, const double *v,
                       int a, int b, double scale, long long n_rows,
                       const long long *rows, double *out)
{
    if (B < 1 || H < 1 || T < 1 || P < 1 || dk < 1 || dv < 1 || a < 1) return ORC_EARG;
    if (kind == 1 && b < 1) return ORC_EARG;
    long long L = (long long)T * P;
    long long total = (long long)B * H * L;
    for (long long r = 0; r < n_rows; ++r)
        if (rows[r] < 0 || rows[r] >= total) return ORC_EARG;
    int status = ORC_OK;
#pragma omp parallel for schedule(dynamic, 4)
    for (long long r = 0; r < n_rows; ++r) {
        long long bh = rows[r] / L;
        long long t = rows[r] % L;
        int f = (int)(t / P);
        int *frames = (int *)malloc(sizeof(int) * (size_t)a);
        if (!frames) { status = ORC_ENOMEM; continue; }
        int nf = (kind == 0) ? swa_frames(f, a, frames) : dswa_frames(f, a, b, frames);
        int st = attend_frames(qrows + r * dk, k + bh * L * dk, v + bh * L * dv,
                               P, dk, dv, frames, nf, scale, out + r * dv);
        if (st != ORC_OK) status = st;
        free(frames);
    }
    return status;
}

/* SWA for the listed query rows ([P1] SWA paragraph); qrows: [n_rows][dk]. */
int oracle_swa_rows(int B, int H, int T, int P, int dk, int dv,
                    const double *qrows, const double *k, const double *v,
                    int window, double scale, long long n_rows,
                    const long long *rows, double *out)
{
    return window_rows(0, B, H, T, P, dk, dv, qrows, k, v, window, 0, scale, n_rows, rows, out);
}

/* DSWA for the listed query rows ([P1] DSWA paragraph); qrows: [n_rows][dk]. */
int oracle_dswa_rows(int B, int H, int T, int P, int dk, int dv,
                     const double *qrows, const double *k, const double *v,
                     int taps, int dilation, double scale, long long n_rows,
                     const long long *rows, double *out)
{
    return window_rows(1, B, H, T, P, dk, dv, qrows, k, v, taps, dilation, scale, n_rows, rows, out);
}

static int window_all(int kind, int B, int H, int T, int P, int dk, int dv,
                      const double *q, const double *k, const double *v,
                      int a, int b, double scale, double *o)
{
    long long n = (long long)B * H * T * P;
    long long *rows = (long long *)malloc(sizeof(long long) * (size_t)(n > 0 ? n : 1));
    if (!rows) return ORC_ENOMEM;
    for (long long r = 0; r < n; ++r) rows[r] = r;
    int st = window_rows(kind, B, H, T, P, dk, dv, q, k, v, a, b, scale, n, rows, o);
    free(rows);
    return st;
}

/* SWA over every token; o is [B][H][L][dv]. */
int oracle_swa(int B, int H, int T, int P, int dk, int dv,
               const double *q, const double *k, const double *v,
               int window, double scale, double *o)
{
    return window_all(0, B, H, T, P, dk, dv, q, k, v, window, 0, scale, o);
}

/* DSWA over every token; o is [B][H][L][dv]. */
int oracle_dswa(int B, int H, int T, int P, int dk, int dv,
                const double *q, const double *k, const double *v,
                int taps, int dilation, double scale, double *o)
{
    return window_all(1, B, H, T, P, dk, dv, q, k, v, taps, dilation, scale, o);
}

/*
 * GLA, token by token ([P1] GLA paragraph and update equations, GatedDeltaNet
 * reading when form == 0; the literal printed form when form == 1).
 *   form 0:  S_t = alpha (S - beta v_old k^T) + beta v k^T
 *   form 1:  v_new = beta v + (1 - beta) v_old;
 *            S_t = alpha S - v_old k^T + v_new k^T
 * In both forms v_old = S_{t-1} k_t and o_t = scale * S_t q_t.
 * state: [B][H][dk][dv] holding S^T; in = S_0, out = S_L. o: [B][H][L][dv].
 */
static int gla_run(int form, int B, int H, long long L, int dk, int dv,
                   const double *q, const double *k, const double *v,
                   const double *alpha, const double *beta, double scale,
                   double *state, double *o)
{
    if (B < 1 || H < 1 || L < 0 || dk < 1 || dv < 1) return ORC_EARG;
    int status = ORC_OK;
#pragma omp parallel for schedule(dynamic, 1)
    for (long long bh = 0; bh < (long long)B * H; ++bh) {
        double *S = (double *)malloc(sizeof(double) * (size_t)dv * dk);  /* S[j][i] */
        double *vold = (double *)malloc(sizeof(double) * (size_t)dv);
        double *vnew = (double *)malloc(sizeof(double) * (size_t)dv);
        if (!S || !vold || !vnew) { status = ORC_ENOMEM; free(S); free(vold); free(vnew); continue; }
        double *st = state + bh * dk * dv;
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j) S[(long)j * dk + i] = st[(long)i * dv + j];
        for (long long t = 0; t < L; ++t) {
            const double *kt = k + (bh * L + t) * dk;
            const double *vt = v + (bh * L + t) * dv;
            const double *qt = q + (bh * L + t) * dk;
            double a = alpha[bh * L + t];
            double b = beta[bh * L + t];
            for (int j = 0; j < dv; ++j) {
                double s = 0.0;
                for (int i = 0; i < dk; ++i) s += S[(long)j * dk + i] * kt[i];
                vold[j] = s;
            }
            if (form == 0) {
                for (int j = 0; j < dv; ++j)
                    for (int i = 0; i < dk; ++i)
                        S[(long)j * dk + i] = a * (S[(long)j * dk + i] - b * vold[j] * kt[i])
                                              + b * vt[j] * kt[i];
            } else {
                for (int j = 0; j < dv; ++j) vnew[j] = b * vt[j] + (1.0 - b) * vold[j];
                for (int j = 0; j < dv; ++j)
                    for (int i = 0; i < dk; ++i)
                        S[(long)j * dk + i] = a * S[(long)j * dk + i] - vold[j] * kt[i]
                                              + vnew[j] * kt[i];
            }
            double *ot = o + (bh * L + t) * dv;
            for (int j = 0; j < dv; ++j) {
                double s = 0.0;
                for (int i = 0; i < dk; ++i) s += S[(long)j * dk + i] * qt[i];
                ot[j] = scale * s;
            }
        }
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j) st[(long)i * dv + j] = S[(long)j * dk + i];
        free(S); free(vold); free(vnew);
    }
    return status;
}

/* GLA, GatedDeltaNet reading (the one the HIP path implements). */
int oracle_gla(int B, int H, long long L, int dk, int dv,
               const double *q, const double *k, const double *v,
               const double *alpha, const double *beta, double scale,
               double *state, double *o)
{
    return gla_run(0, B, H, L, dk, dv, q, k, v, alpha, beta, scale, state, o);
}

/* GLA, the three update lines exactly as printed in [P1]. */
int oracle_gla_literal(int B, int H, long long L, int dk, int dv,
                       const double *q, const double *k, const double *v,
                       const double *alpha, const double *beta, double scale,
                       double *state, double *o)
{
    return gla_run(1, B, H, L, dk, dv, q, k, v, alpha, beta, scale, state, o);
}

/* Threads the parallel loops above use (the OpenMP team size). */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
