/*
 * KDA oracle R-bwd: the gradient of the token-by-token recurrence, in double
 * precision (reverse-mode adjoint of oracle R).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file.  It shares no code, header or constant with the GPU
 * library.
 *
 * The forward recurrence is the one of kda_recurrence.c ("You could have
 * come up with Kimi Delta Attention", the five state-update equations at
 * the top; GeekNews #31925, section "Kimi Delta Attention: per-channel
 * decay"), with the transposed state H = S^T (Dk x Dv):
 *
 *   Ht~ = Diag(alpha_t) H_{t-1}       alpha_t = exp(g_t)
 *   p   = Ht~^T k_t                    (prediction S~_t k_t)
 *   e   = beta_t (v_t - p)
 *   H_t = Ht~ + k_t e^T
 *   o_t = H_t^T (scale q_t)
 *
 * The training signal is a scalar loss L whose gradients dL/do_t (dO) and
 * dL/dH_T (dHT, optional) are given; the pages say the method is trained
 * with the chunkwise algorithm (F29 course outline, "Paper: Gated DeltaNet ->
 * Kimi Delta Attention"; GeekNews #31925, section "Fused recurrent kernel
 * for decode": the chunkwise form serves training).  Reverse mode walks the
 * five steps backwards, t = T-1 .. 0, carrying D = dL/dH_t:
 *
 *   read     dq_t = scale H_t dO_t ;            D += scale q_t dO_t^T
 *   write    de = D^T k_t ; dk_t = D e ;        (Ht~ receives D)
 *   correct  dv_t = beta_t de ; dbeta_t = de . (v_t - p) ; dp = -beta_t de
 *   predict  dk_t += Ht~ dp ;                   D += k_t dp^T
 *   forget   dg_t[c] = alpha_t[c] sum_j H_{t-1}[c][j] D[c][j] ;  D = Diag(alpha_t) D
 *
 * leaving D = dL/dH_{-1}, the gradient of the initial state.  The scalar-gate
 * mode sums the forget-step product over the whole state; the ungated mode
 * has no gate gradient.  States H_{t-1} are recomputed per segment of 64
 * tokens from checkpoints taken during one forward sweep.
 *
 * Layouts (contiguous doubles, as in kda_recurrence.c):
 *   q, k, dq, dk [B,T,H,Dk]   v, dO, dv [B,T,H,Dv]   beta, dbeta [B,T,H]
 *   g, dg   mode 0 [B,T,H,Dk]; mode 1 [B,T,H]; mode 2 unused (dg may be NULL)
 *   h0, dhT, dh0  [B,H,Dk,Dv] or NULL (zero / not stored)
 *
 * Returns 0 on success, -1 on bad arguments, -2 on allocation failure.
 * KDA_MUTANT >= 101 selects a deliberately wrong gradient (tests only).
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#ifndef KDA_MUTANT
#define KDA_MUTANT 0
#endif

enum { BWD_CHANNEL = 0, BWD_SCALAR = 1, BWD_NONE = 2 };
enum { SEG = 64 };

/* Forget step on the transposed state: rows (key channels) scaled. */
static void forget(double* Hs, const double* g, long tok, long Dk, long Dv, int mode)
{
    if (mode == BWD_CHANNEL) {
        for (long c = 0; c < Dk; ++c) {
            const double a = exp(g[tok * Dk + c]);
            for (long j = 0; j < Dv; ++j) Hs[c * Dv + j] *= a;
        }
    } else if (mode == BWD_SCALAR) {
        const double a = exp(g[tok]);
        for (long i = 0; i < Dk * Dv; ++i) Hs[i] *= a;
    }
}

/* One forward token: Hs holds H_{t-1} on entry and H_t on exit; p and e get
 * the prediction and the error. */
static void step(double* Hs, const double* kt, const double* vt, double bt,
                 const double* g, long tok, long Dk, long Dv, int mode,
                 double* p, double* e)
{
    forget(Hs, g, tok, Dk, Dv, mode);
    for (long j = 0; j < Dv; ++j) p[j] = 0.0;
    for (long c = 0; c < Dk; ++c)
        for (long j = 0; j < Dv; ++j) p[j] += Hs[c * Dv + j] * kt[c];
    for (long j = 0; j < Dv; ++j) e[j] = bt * (vt[j] - p[j]);
    for (long c = 0; c < Dk; ++c)
        for (long j = 0; j < Dv; ++j) Hs[c * Dv + j] += kt[c] * e[j];
}

typedef struct {
    const double *q, *k, *v, *g, *beta, *h0, *dO, *dhT;
    double *dq, *dk, *dv, *dg, *dbeta, *dh0;
    long B, T, H, Dk, Dv;
    double scale;
    int mode;
} bwd_args;

static int one_sequence(const bwd_args* a, long b, long h, double* work)
{
    const long Dk = a->Dk, Dv = a->Dv, T = a->T, H = a->H, DD = Dk * Dv;
    const long nseg = (T + SEG - 1) / SEG;
    double* ck = work;                    /* nseg checkpoints: H before each segment */
    double* seg = ck + nseg * DD;         /* SEG states H_{t-1} of the current segment */
    double* Hs = seg + SEG * DD;          /* running state */
    double* Ht = Hs + DD;                 /* H~ of the current token */
    double* D = Ht + DD;                  /* adjoint dL/dH */
    double* p = D + DD;
    double* e = p + Dv;
    double* de = e + Dv;
    double* dp = de + Dv;
    const long unit = b * H + h;

    /* forward sweep: checkpoints only */
    if (a->h0) memcpy(Hs, a->h0 + unit * DD, sizeof(double) * DD);
    else memset(Hs, 0, sizeof(double) * DD);
    for (long t = 0; t < T; ++t) {
        if (t % SEG == 0) memcpy(ck + (t / SEG) * DD, Hs, sizeof(double) * DD);
        const long tok = (b * T + t) * H + h;
        step(Hs, a->k + tok * Dk, a->v + tok * Dv, a->beta[tok], a->g, tok, Dk, Dv,
             a->mode, p, e);
    }

    if (a->dhT) memcpy(D, a->dhT + unit * DD, sizeof(double) * DD);
    else memset(D, 0, sizeof(double) * DD);

    for (long s = nseg - 1; s >= 0; --s) {
        const long t0 = s * SEG, t1 = (t0 + SEG < T) ? t0 + SEG : T;
        /* recompute H_{t-1} for t in [t0, t1) */
        memcpy(Hs, ck + s * DD, sizeof(double) * DD);
        for (long t = t0; t < t1; ++t) {
            memcpy(seg + (t - t0) * DD, Hs, sizeof(double) * DD);
            const long tok = (b * T + t) * H + h;
            step(Hs, a->k + tok * Dk, a->v + tok * Dv, a->beta[tok], a->g, tok, Dk, Dv,
                 a->mode, p, e);
        }
        for (long t = t1 - 1; t >= t0; --t) {
            const long tok = (b * T + t) * H + h;
            const double* kt = a->k + tok * Dk;
            const double* qt = a->q + tok * Dk;
            const double* vt = a->v + tok * Dv;
            const double* dot = a->dO + tok * Dv;
            const double bt = a->beta[tok];
            const double* Hprev = seg + (t - t0) * DD;
            double* dqt = a->dq + tok * Dk;
            double* dkt = a->dk + tok * Dk;
            double* dvt = a->dv + tok * Dv;

            /* rebuild H~, p, e and H_t (into Hs) for this token */
            memcpy(Ht, Hprev, sizeof(double) * DD);
            forget(Ht, a->g, tok, Dk, Dv, a->mode);
            for (long j = 0; j < Dv; ++j) p[j] = 0.0;
            for (long c = 0; c < Dk; ++c)
                for (long j = 0; j < Dv; ++j) p[j] += Ht[c * Dv + j] * kt[c];
            for (long j = 0; j < Dv; ++j) e[j] = bt * (vt[j] - p[j]);
            for (long c = 0; c < Dk; ++c)
                for (long j = 0; j < Dv; ++j) Hs[c * Dv + j] = Ht[c * Dv + j] + kt[c] * e[j];

            /* read: o_t = H_t^T (scale q_t) */
            for (long c = 0; c < Dk; ++c) {
                double acc = 0.0;
#if KDA_MUTANT == 101
                /* mutant: query gradient taken from the state before the write */
                for (long j = 0; j < Dv; ++j) acc += Ht[c * Dv + j] * dot[j];
#else
                for (long j = 0; j < Dv; ++j) acc += Hs[c * Dv + j] * dot[j];
#endif
                dqt[c] = a->scale * acc;
            }
            for (long c = 0; c < Dk; ++c)
                for (long j = 0; j < Dv; ++j) D[c * Dv + j] += a->scale * qt[c] * dot[j];

            /* write: H_t = H~ + k e^T */
            for (long j = 0; j < Dv; ++j) {
                double acc = 0.0;
                for (long c = 0; c < Dk; ++c) acc += kt[c] * D[c * Dv + j];
                de[j] = acc;
            }
            for (long c = 0; c < Dk; ++c) {
                double acc = 0.0;
                for (long j = 0; j < Dv; ++j) acc += D[c * Dv + j] * e[j];
                dkt[c] = acc;
            }

            /* correct: e = beta (v - p) */
            double db = 0.0;
            for (long j = 0; j < Dv; ++j) {
                dvt[j] = bt * de[j];
                db += de[j] * (vt[j] - p[j]);
#if KDA_MUTANT == 102
                dp[j] = bt * de[j];                /* mutant: sign of the prediction path */
#else
                dp[j] = -bt * de[j];
#endif
            }
            a->dbeta[tok] = db;

            /* predict: p = H~^T k */
            for (long c = 0; c < Dk; ++c) {
                double acc = 0.0;
                for (long j = 0; j < Dv; ++j) acc += Ht[c * Dv + j] * dp[j];
#if KDA_MUTANT == 103
                (void)acc;                          /* mutant: key gradient of the prediction dropped */
#else
                dkt[c] += acc;
#endif
            }
            for (long c = 0; c < Dk; ++c)
                for (long j = 0; j < Dv; ++j) D[c * Dv + j] += kt[c] * dp[j];

            /* forget: H~ = Diag(alpha) H_{t-1} */
            if (a->mode == BWD_CHANNEL) {
                for (long c = 0; c < Dk; ++c) {
                    const double al = exp(a->g[tok * Dk + c]);
                    double acc = 0.0;
                    for (long j = 0; j < Dv; ++j) acc += Hprev[c * Dv + j] * D[c * Dv + j];
#if KDA_MUTANT == 104
                    a->dg[tok * Dk + c] = acc;          /* mutant: chain factor alpha dropped */
#else
                    a->dg[tok * Dk + c] = al * acc;
#endif
#if KDA_MUTANT != 105
                    for (long j = 0; j < Dv; ++j) D[c * Dv + j] *= al;
#endif
                }
            } else if (a->mode == BWD_SCALAR) {
                const double al = exp(a->g[tok]);
                double acc = 0.0;
                for (long i = 0; i < DD; ++i) acc += Hprev[i] * D[i];
                a->dg[tok] = al * acc;
#if KDA_MUTANT != 105
                for (long i = 0; i < DD; ++i) D[i] *= al;   /* mutant 105: adjoint not decayed */
#endif
            }
        }
    }
    if (a->dh0) memcpy(a->dh0 + unit * DD, D, sizeof(double) * DD);
    return 0;
}

int kda_oracle_recurrent_bwd(const double* q, const double* k, const double* v,
                             const double* g, const double* beta, const double* h0,
                             const double* dO, const double* dhT,
                             double* dq, double* dk, double* dv, double* dg,
                             double* dbeta, double* dh0,
                             long B, long T, long H, long Dk, long Dv,
                             double scale, int mode, int nthreads)
{
    if (!q || !k || !v || !beta || !dO || !dq || !dk || !dv || !dbeta)
        return -1;
    if (B < 0 || T < 0 || H < 0 || Dk <= 0 || Dv <= 0)
        return -1;
    if (mode != BWD_CHANNEL && mode != BWD_SCALAR && mode != BWD_NONE)
        return -1;
    if (mode != BWD_NONE && (!g || !dg))
        return -1;
    bwd_args a = {q, k, v, g, beta, h0, dO, dhT, dq, dk, dv, dg, dbeta, dh0,
                  B, T, H, Dk, Dv, scale, mode};
    const long units = B * H;
    const long nseg = (T + SEG - 1) / SEG;
    const long words = (nseg + SEG + 3) * Dk * Dv + 4 * Dv;
    int failed = 0;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel num_threads(nthreads) reduction(| : failed)
#endif
    {
        double* work = (double*)malloc(sizeof(double) * words);
        if (!work) failed = 1;
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
        for (long u = 0; u < units; ++u) {
            if (!work) continue;
            one_sequence(&a, u / H, u % H, work);
        }
        free(work);
    }
    return failed ? -2 : 0;
}
