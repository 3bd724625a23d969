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

/* ------------------------------------------------------------------------ */
/* Backward pass: the exact gradient of the forward definitions above.       */
/*                                                                          */
/* The pages train the model built from these layers (the curriculum over    */
/* 81- and 241-frame clips in [P1] section 二、方法), so each layer also needs  */
/* its vector-Jacobian product: given dO = dL/dO, return dL/dq, dL/dk, dL/dv  */
/* (and, for GLA, dL/dalpha, dL/dbeta and dL/dS_0). Nothing here is taken     */
/* from the pages beyond the forward definitions; the rules are the chain     */
/* rule written out.                                                        */
/* ------------------------------------------------------------------------ */

/*
 * Softmax statistics of one query row over its window: log-sum-exp of the
 * scaled logits, and D = dO_t . o_t (the row's output dotted with its output
 * gradient). Used by the backward rules
 *   p_s  = exp(z_s - lse),  dp_s = dO_t . v_s,  ds_s = p_s (dp_s - D),
 *   dq_t = scale sum_s ds_s k_s,  dk_s += scale ds_s q_t,  dv_s += p_s dO_t.
 */
static int row_stats(const double *qrow, const double *dorow, const double *kbh,
                     const double *vbh, int P, int dk, int dv, const int *frames, int nf,
                     double scale, double *lse_out, double *D_out)
{
    double *o = (double *)malloc(sizeof(double) * (size_t)dv);
    if (!o) return ORC_ENOMEM;
    int st = attend_frames(qrow, kbh, vbh, P, dk, dv, frames, nf, scale, o);
    if (st == ORC_OK) {
        double m = -INFINITY;
        for (int a = 0; a < nf; ++a)
            for (int p = 0; p < P; ++p) {
                const double *kr = kbh + ((long)frames[a] * P + p) * dk;
                double s = 0.0;
                for (int i = 0; i < dk; ++i) s += qrow[i] * kr[i];
                s *= scale;
                if (s > m) m = s;
            }
        double den = 0.0;
        for (int a = 0; a < nf; ++a)
            for (int p = 0; p < P; ++p) {
                const double *kr = kbh + ((long)frames[a] * P + p) * dk;
                double s = 0.0;
                for (int i = 0; i < dk; ++i) s += qrow[i] * kr[i];
                den += exp(s * scale - m);
            }
        *lse_out = m + log(den);
        double D = 0.0;
        for (int j = 0; j < dv; ++j) D += dorow[j] * o[j];
        *D_out = D;
    }
    free(o);
    return st;
}

static int window_frames(int kind, int f, int a, int b, int *frames)
{
    return (kind == 0) ? swa_frames(f, a, frames) : dswa_frames(f, a, b, frames);
}

/*
 * Full backward of SWA (kind 0, a = window) or DSWA (kind 1, a = taps,
 * b = dilation) over every token. Parallel over (batch, head); inside one
 * slice the query rows run in order and scatter into dk, dv.
 */
static int window_bwd(int kind, int B, int H, int T, int P, int dk, int dv,
                      const double *q, const double *k, const double *v, const double *dout,
                      int a, int b, double scale, double *dq, double *dkk, double *dvv)
{
    if (B < 1 || H < 1 || T < 1 || P < 1 || dk < 1 || dv < 1 || a < 1) return ORC_EARG;
    if (kind == 1 && b < 1) return ORC_EARG;
    const long long L = (long long)T * P;
    int status = ORC_OK;
#pragma omp parallel for schedule(dynamic, 1)
    for (long long bh = 0; bh < (long long)B * H; ++bh) {
        const double *qb = q + bh * L * dk, *kb = k + bh * L * dk, *vb = v + bh * L * dv;
        const double *dob = dout + bh * L * dv;
        double *dqb = dq + bh * L * dk, *dkb = dkk + bh * L * dk, *dvb = dvv + bh * L * dv;
        int *frames = (int *)malloc(sizeof(int) * (size_t)a);
        if (!frames) { status = ORC_ENOMEM; continue; }
        for (long long e = 0; e < L * dk; ++e) { dqb[e] = 0.0; dkb[e] = 0.0; }
        for (long long e = 0; e < L * dv; ++e) dvb[e] = 0.0;
        for (long long t = 0; t < L; ++t) {
            const double *qt = qb + t * dk, *dot = dob + t * dv;
            int nf = window_frames(kind, (int)(t / P), a, b, frames);
            double lse, D;
            int st = row_stats(qt, dot, kb, vb, P, dk, dv, frames, nf, scale, &lse, &D);
            if (st != ORC_OK) { status = st; break; }
            for (int f = 0; f < nf; ++f)
                for (int p = 0; p < P; ++p) {
                    long long s = (long long)frames[f] * P + p;
                    const double *ks = kb + s * dk, *vs = vb + s * dv;
                    double z = 0.0, dp = 0.0;
                    for (int i = 0; i < dk; ++i) z += qt[i] * ks[i];
                    for (int j = 0; j < dv; ++j) dp += dot[j] * vs[j];
                    double pr = exp(z * scale - lse);
                    double ds = pr * (dp - D);
                    for (int i = 0; i < dk; ++i) {
                        dqb[t * dk + i] += scale * ds * ks[i];
                        dkb[s * dk + i] += scale * ds * qt[i];
                    }
                    for (int j = 0; j < dv; ++j) dvb[s * dv + j] += pr * dot[j];
                }
        }
        free(frames);
    }
    return status;
}

int oracle_swa_bwd(int B, int H, int T, int P, int dk, int dv,
                   const double *q, const double *k, const double *v, const double *dout,
                   int window, double scale, double *dq, double *dkk, double *dvv)
{
    return window_bwd(0, B, H, T, P, dk, dv, q, k, v, dout, window, 0, scale, dq, dkk, dvv);
}

int oracle_dswa_bwd(int B, int H, int T, int P, int dk, int dv,
                    const double *q, const double *k, const double *v, const double *dout,
                    int taps, int dilation, double scale, double *dq, double *dkk, double *dvv)
{
    return window_bwd(1, B, H, T, P, dk, dv, q, k, v, dout, taps, dilation, scale, dq, dkk, dvv);
}

/*
 * Per-row statistics (lse, D) for listed flat query rows; the query and
 * output-gradient vectors of those rows are passed compactly ([n][dk], [n][dv]).
 */
int oracle_window_stats(int kind, int B, int H, int T, int P, int dk, int dv,
                        const double *qrows, const double *dorows,
                        const double *k, const double *v, int a, int b, double scale,
                        long long n_rows, const long long *rows, double *lse, double *D)
{
    if (B < 1 || H < 1 || T < 1 || P < 1 || dk < 1 || dv < 1 || a < 1) return ORC_EARG;
    if (kind == 1 && b < 1) return ORC_EARG;
    const long long L = (long long)T * P, total = (long long)B * H * L;
    for (long long r = 0; r < n_rows; ++r)
        if (rows[r] < 0 || rows[r] >= total) return ORC_EARG;
    int status = ORC_OK;
#pragma omp parallel for schedule(dynamic, 4)
    for (long long r = 0; r < n_rows; ++r) {
        long long bh = rows[r] / L, t = rows[r] % L;
        int *frames = (int *)malloc(sizeof(int) * (size_t)a);
        if (!frames) { status = ORC_ENOMEM; continue; }
        int nf = window_frames(kind, (int)(t / P), a, b, frames);
        int st = row_stats(qrows + r * dk, dorows + r * dv, k + bh * L * dk, v + bh * L * dv,
                           P, dk, dv, frames, nf, scale, lse + r, D + r);
        if (st != ORC_OK) status = st;
        free(frames);
    }
    return status;
}

/*
 * dq for listed flat query rows (row-local: the row's whole window).
 * qrows, dorows: [n][dk], [n][dv]; dq_out: [n][dk].
 */
int oracle_window_dq_rows(int kind, int B, int H, int T, int P, int dk, int dv,
                          const double *qrows, const double *dorows,
                          const double *k, const double *v, int a, int b, double scale,
                          long long n_rows, const long long *rows, double *dq_out)
{
    if (B < 1 || H < 1 || T < 1 || P < 1 || dk < 1 || dv < 1 || a < 1) return ORC_EARG;
    if (kind == 1 && b < 1) return ORC_EARG;
    const long long L = (long long)T * P, total = (long long)B * H * L;
    for (long long r = 0; r < n_rows; ++r)
        if (rows[r] < 0 || rows[r] >= total) return ORC_EARG;
    int status = ORC_OK;
#pragma omp parallel for schedule(dynamic, 4)
    for (long long r = 0; r < n_rows; ++r) {
        long long bh = rows[r] / L, t = rows[r] % L;
        const double *kb = k + bh * L * dk, *vb = v + bh * L * dv;
        const double *qt = qrows + r * dk, *dot = dorows + r * dv;
        double *dqt = dq_out + r * dk;
        int *frames = (int *)malloc(sizeof(int) * (size_t)a);
        if (!frames) { status = ORC_ENOMEM; continue; }
        int nf = window_frames(kind, (int)(t / P), a, b, frames);
        double lse, D;
        int st = row_stats(qt, dot, kb, vb, P, dk, dv, frames, nf, scale, &lse, &D);
        for (int i = 0; i < dk; ++i) dqt[i] = 0.0;
        if (st != ORC_OK) { status = st; free(frames); continue; }
        for (int f = 0; f < nf; ++f)
            for (int p = 0; p < P; ++p) {
                long long s = (long long)frames[f] * P + p;
                const double *ks = kb + s * dk, *vs = vb + s * dv;
                double z = 0.0, dp = 0.0;
                for (int i = 0; i < dk; ++i) z += qt[i] * ks[i];
                for (int j = 0; j < dv; ++j) dp += dot[j] * vs[j];
                double ds = exp(z * scale - lse) * (dp - D);
                for (int i = 0; i < dk; ++i) dqt[i] += scale * ds * ks[i];
            }
        free(frames);
    }
    return status;
}

/*
 * dk, dv for listed flat key rows: sum over every query whose window holds the
 * key's frame. lse and D are per-row statistics laid out [B*H*L]; only the
 * entries of those queries are read. dk_out: [n][dk], dv_out: [n][dv].
 */
int oracle_window_dkv_rows(int kind, int B, int H, int T, int P, int dk, int dv,
                           const double *q, const double *k, const double *v,
                           const double *dout, const double *lse, const double *D,
                           int a, int b, double scale, long long n_rows,
                           const long long *rows, double *dk_out, double *dv_out)
{
    if (B < 1 || H < 1 || T < 1 || P < 1 || dk < 1 || dv < 1 || a < 1) return ORC_EARG;
    if (kind == 1 && b < 1) return ORC_EARG;
    const long long L = (long long)T * P, total = (long long)B * H * L;
    for (long long r = 0; r < n_rows; ++r)
        if (rows[r] < 0 || rows[r] >= total) return ORC_EARG;
    const int step = (kind == 0) ? 1 : b;
#pragma omp parallel for schedule(dynamic, 4)
    for (long long r = 0; r < n_rows; ++r) {
        long long bh = rows[r] / L, s = rows[r] % L;
        int kf = (int)(s / P);
        const double *ks = k + rows[r] * dk, *vs = v + rows[r] * dv;
        double *dks = dk_out + r * dk, *dvs = dv_out + r * dv;
        for (int i = 0; i < dk; ++i) dks[i] = 0.0;
        for (int j = 0; j < dv; ++j) dvs[j] = 0.0;
        /* query frames whose window holds frame kf: kf + j*step, j < a */
        for (int j = 0; j < a; ++j) {
            long long fq = (long long)kf + (long long)j * step;
            if (fq >= T) break;
            for (int p = 0; p < P; ++p) {
                long long t = bh * L + fq * P + p;
                const double *qt = q + t * dk, *dot = dout + t * dv;
                double z = 0.0, dp = 0.0;
                for (int i = 0; i < dk; ++i) z += qt[i] * ks[i];
                for (int jj = 0; jj < dv; ++jj) dp += dot[jj] * vs[jj];
                double pr = exp(z * scale - lse[t]);
                double ds = pr * (dp - D[t]);
                for (int i = 0; i < dk; ++i) dks[i] += scale * ds * qt[i];
                for (int jj = 0; jj < dv; ++jj) dvs[jj] += pr * dot[jj];
            }
        }
    }
    return ORC_OK;
}

/*
 * GLA backward, token by token in reverse (form 0: GatedDeltaNet reading,
 * form 1: the printed update). With M = S^T (dk x dv) and u = M_{t-1}^T k_t:
 *   form 0:  M_t = alpha M_{t-1} - alpha beta k u^T + beta k v^T
 *   form 1:  M_t = alpha M_{t-1} -       beta k u^T + beta k v^T
 *   o_t = scale M_t^T q_t.
 * G holds dL/dM_t while walking t = L-1 .. 0:
 *   G += scale q_t dO_t^T;  dq_t = scale M_t dO_t;  w = G^T k_t
 *   dv_t = beta w
 *   form 0: dalpha = <G, M_{t-1} - beta k u^T>, dbeta = w.(v - alpha u),
 *           du = -alpha beta w, dk_t = beta G (v - alpha u) + M_{t-1} du
 *   form 1: dalpha = <G, M_{t-1}>, dbeta = w.(v - u),
 *           du = -beta w, dk_t = beta G (v - u) + M_{t-1} du
 *   G <- alpha G + k du^T   (dL/dM_{t-1})
 * dstate_final (dL/dM_L, may be NULL = 0) seeds G; dstate0 receives dL/dM_0.
 * The forward states are recomputed from checkpoints every `ck` tokens.
 */
static int gla_bwd_run(int form, int B, int H, long long L, int dk, int dv,
                       const double *q, const double *k, const double *v,
                       const double *alpha, const double *beta, double scale,
                       const double *state0, const double *dout, const double *dstate_final,
                       double *dq, double *dkk, double *dvv, double *dalpha, double *dbeta,
                       double *dstate0)
{
    if (B < 1 || H < 1 || L < 0 || dk < 1 || dv < 1) return ORC_EARG;
    const long long ck = 64;
    const long long nck = (L + ck - 1) / ck;
    const long long DD = (long long)dk * dv;
    int status = ORC_OK;
#pragma omp parallel for schedule(dynamic, 1)
    for (long long bh = 0; bh < (long long)B * H; ++bh) {
        double *cks = (double *)malloc(sizeof(double) * (size_t)((nck + 1) * DD));
        double *seg = (double *)malloc(sizeof(double) * (size_t)((ck + 1) * DD));
        double *G = (double *)malloc(sizeof(double) * (size_t)DD);
        double *u = (double *)malloc(sizeof(double) * (size_t)dv);
        double *w = (double *)malloc(sizeof(double) * (size_t)dv);
        double *du = (double *)malloc(sizeof(double) * (size_t)dv);
        if (!cks || !seg || !G || !u || !w || !du) {
            status = ORC_ENOMEM;
            free(cks); free(seg); free(G); free(u); free(w); free(du);
            continue;
        }
        const double *qb = q + bh * L * dk, *kb = k + bh * L * dk, *vb = v + bh * L * dv;
        const double *ab = alpha + bh * L, *bb = beta + bh * L, *dob = dout + bh * L * dv;
        /* forward pass, keeping M at every checkpoint (M_0, M_ck, ...) */
        memcpy(cks, state0 + bh * DD, sizeof(double) * (size_t)DD);
        double *M = seg;
        memcpy(M, cks, sizeof(double) * (size_t)DD);
        for (long long t = 0; t < L; ++t) {
            const double *kt = kb + t * dk, *vt = vb + t * dv;
            const double a = ab[t], be = bb[t];
            for (int j = 0; j < dv; ++j) {
                double s = 0.0;
                for (int i = 0; i < dk; ++i) s += M[(long)i * dv + j] * kt[i];
                u[j] = s;
            }
            const double ea = (form == 0) ? a * be : be;
            for (int i = 0; i < dk; ++i)
                for (int j = 0; j < dv; ++j)
                    M[(long)i * dv + j] = a * M[(long)i * dv + j] - ea * kt[i] * u[j]
                                          + be * kt[i] * vt[j];
            if ((t + 1) % ck == 0 && (t + 1) / ck <= nck)
                memcpy(cks + ((t + 1) / ck) * DD, M, sizeof(double) * (size_t)DD);
        }
        /* reverse pass */
        for (long long e = 0; e < DD; ++e)
            G[e] = dstate_final ? dstate_final[bh * DD + e] : 0.0;
        for (long long c = nck - 1; c >= 0; --c) {
            const long long t0 = c * ck, t1 = (t0 + ck < L) ? t0 + ck : L;
            /* recompute M_{t0} .. M_{t1} of this segment into seg[0 .. t1-t0] */
            memcpy(seg, cks + c * DD, sizeof(double) * (size_t)DD);
            for (long long t = t0; t < t1; ++t) {
                const double *Mp = seg + (t - t0) * DD;
                double *Mn = seg + (t - t0 + 1) * DD;
                const double *kt = kb + t * dk, *vt = vb + t * dv;
                const double a = ab[t], be = bb[t];
                for (int j = 0; j < dv; ++j) {
                    double s = 0.0;
                    for (int i = 0; i < dk; ++i) s += Mp[(long)i * dv + j] * kt[i];
                    u[j] = s;
                }
                const double ea = (form == 0) ? a * be : be;
                for (int i = 0; i < dk; ++i)
                    for (int j = 0; j < dv; ++j)
                        Mn[(long)i * dv + j] = a * Mp[(long)i * dv + j] - ea * kt[i] * u[j]
                                               + be * kt[i] * vt[j];
            }
            for (long long t = t1 - 1; t >= t0; --t) {
                const double *Mp = seg + (t - t0) * DD;      /* M_{t-1} */
                const double *Mt = seg + (t - t0 + 1) * DD;  /* M_t */
                const double *qt = qb + t * dk, *kt = kb + t * dk, *vt = vb + t * dv;
                const double *dot = dob + t * dv;
                const double a = ab[t], be = bb[t];
                double *dqt = dq + (bh * L + t) * dk, *dkt = dkk + (bh * L + t) * dk;
                double *dvt = dvv + (bh * L + t) * dv;
                for (int i = 0; i < dk; ++i) {
                    double s = 0.0;
                    for (int j = 0; j < dv; ++j) {
                        G[(long)i * dv + j] += scale * qt[i] * dot[j];
                        s += Mt[(long)i * dv + j] * dot[j];
                    }
                    dqt[i] = scale * s;
                }
                for (int j = 0; j < dv; ++j) {
                    double s = 0.0, s2 = 0.0;
                    for (int i = 0; i < dk; ++i) {
                        s += G[(long)i * dv + j] * kt[i];
                        s2 += Mp[(long)i * dv + j] * kt[i];
                    }
                    w[j] = s;
                    u[j] = s2;
                }
                const double ua = (form == 0) ? a : 1.0;   /* u enters as ua * u */
                double da = 0.0, db = 0.0;
                for (int i = 0; i < dk; ++i)
                    for (int j = 0; j < dv; ++j) {
                        double erase = (form == 0) ? be * kt[i] * u[j] : 0.0;
                        da += G[(long)i * dv + j] * (Mp[(long)i * dv + j] - erase);
                    }
                for (int j = 0; j < dv; ++j) {
                    db += w[j] * (vt[j] - ua * u[j]);
                    dvt[j] = be * w[j];
                    du[j] = -ua * be * w[j];
                }
                for (int i = 0; i < dk; ++i) {
                    double s = 0.0;
                    for (int j = 0; j < dv; ++j)
                        s += G[(long)i * dv + j] * be * (vt[j] - ua * u[j])
                             + Mp[(long)i * dv + j] * du[j];
                    dkt[i] = s;
                }
                dalpha[bh * L + t] = da;
                dbeta[bh * L + t] = db;
                for (int i = 0; i < dk; ++i)
                    for (int j = 0; j < dv; ++j)
                        G[(long)i * dv + j] = a * G[(long)i * dv + j] + kt[i] * du[j];
            }
        }
        memcpy(dstate0 + bh * DD, G, sizeof(double) * (size_t)DD);
        free(cks); free(seg); free(G); free(u); free(w); free(du);
    }
    return status;
}

int oracle_gla_bwd(int form, int B, int H, long long L, int dk, int dv,
                   const double *q, const double *k, const double *v,
                   const double *alpha, const double *beta, double scale,
                   const double *state0, const double *dout, const double *dstate_final,
                   double *dq, double *dkk, double *dvv, double *dalpha, double *dbeta,
                   double *dstate0)
{
    if (form != 0 && form != 1) return ORC_EARG;
    return gla_bwd_run(form, B, H, L, dk, dv, q, k, v, alpha, beta, scale, state0, dout,
                       dstate_final, dq, dkk, dvv, dalpha, dbeta, dstate0);
}
