/*
 * KDA oracle R: the token-by-token recurrence, in double precision.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the reference that the HIP kernels
 * are checked against; nothing on the product path may link, load or call it.
 * It shares no code, header or constant with the GPU library.
 *
 * What it computes, per (batch b, head h), for t = 0 .. T-1
 * ("You could have come up with Kimi Delta Attention", the five state-update
 * equations at the top of the article; GeekNews #31925 section
 * "Kimi Delta Attention: per-channel decay", steps 1-5):
 *
 *   1. forget   Ht~ = Diag(alpha_t) H          alpha_t = exp(g_t)
 *   2. predict  vhat = Ht~^T k_t               (= S~_t k_t)
 *   3. correct  e    = beta_t (v_t - vhat)
 *   4. write    H    = Ht~ + k_t e^T           (= S~_t + e_t k_t^T, transposed)
 *   5. read     o_t  = H^T (scale * q_t)       (= S_t (d_k^-1/2 q_t))
 *
 * H is the state transposed, H = S^T in R^{Dk x Dv}: row = key channel,
 * column = value channel, so the per-channel decay Diag(alpha) scales rows.
 * The scalar-gate mode (Gated DeltaNet, GeekNews #31925 section "Gated
 * DeltaNet: forget the whole state first") multiplies the whole state by one
 * exp(g_t); the ungated mode (DeltaNet, section "DeltaNet: write the error,
 * not the value") skips step 1.  The order forget -> predict -> correct ->
 * write is the one that section insists on.
 *
 * Layouts (all contiguous, doubles):
 *   q, k  [B,T,H,Dk]   v, o [B,T,H,Dv]   beta [B,T,H]
 *   g     mode 0 (channel) [B,T,H,Dk]; mode 1 (scalar) [B,T,H]; mode 2: unused
 *   h0    [B,H,Dk,Dv] or NULL (zero state)   hT [B,H,Dk,Dv] or NULL
 *
 * Returns 0 on success, -1 on bad arguments, -2 on allocation failure.
 *
 * Built with plain -O2 (no fast-math).  KDA_MUTANT selects a deliberately
 * wrong variant; it exists only so the tests can show that the pins catch
 * each plausible mistake, and is never defined in the oracle proper.
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

enum { ORACLE_CHANNEL = 0, ORACLE_SCALAR = 1, ORACLE_NONE = 2 };

static void one_sequence(const double* q, const double* k, const double* v,
                         const double* g, const double* beta, const double* h0,
                         double* o, double* hT, long b, long h,
                         long T, long H, long Dk, long Dv, double scale, int mode,
                         double* S, double* vhat, double* e)
{
    if (h0)
        memcpy(S, h0 + (b * H + h) * Dk * Dv, sizeof(double) * Dk * Dv);
    else
        memset(S, 0, sizeof(double) * Dk * Dv);

    for (long t = 0; t < T; ++t) {
        const long tok = (b * T + t) * H + h;
        const double* kt = k + tok * Dk;
        const double* qt = q + tok * Dk;
        const double* vt = v + tok * Dv;
        const double bt = beta[tok];
        double* ot = o + tok * Dv;

#if KDA_MUTANT == 1
        /* mutant: predict before the forget step */
        for (long j = 0; j < Dv; ++j) vhat[j] = 0.0;
        for (long c = 0; c < Dk; ++c)
            for (long j = 0; j < Dv; ++j) vhat[j] += S[c * Dv + j] * kt[c];
#endif
        /* 1. forget */
        if (mode == ORACLE_CHANNEL) {
            for (long c = 0; c < Dk; ++c) {
#if KDA_MUTANT == 2
                /* mutant: gate indexed by value channel (columns) */
                for (long j = 0; j < Dv; ++j) S[c * Dv + j] *= exp(g[tok * Dk + (j % Dk)]);
#else
                const double a = exp(g[tok * Dk + c]);
                for (long j = 0; j < Dv; ++j) S[c * Dv + j] *= a;
#endif
            }
        } else if (mode == ORACLE_SCALAR) {
            const double a = exp(g[tok]);
            for (long i = 0; i < Dk * Dv; ++i) S[i] *= a;
        }

#if KDA_MUTANT != 1
        /* 2. predict: vhat = S~ k = H~^T k */
        for (long j = 0; j < Dv; ++j) vhat[j] = 0.0;
        for (long c = 0; c < Dk; ++c)
            for (long j = 0; j < Dv; ++j) vhat[j] += S[c * Dv + j] * kt[c];
#endif

        /* 3. correct */
        for (long j = 0; j < Dv; ++j) {
#if KDA_MUTANT == 3
            e[j] = (vt[j] - vhat[j]);              /* mutant: beta dropped */
#elif KDA_MUTANT == 4
            e[j] = bt * (vhat[j] - vt[j]);         /* mutant: sign flipped */
#else
            e[j] = bt * (vt[j] - vhat[j]);
#endif
        }

#if KDA_MUTANT == 5
        /* mutant: read before the write */
        for (long j = 0; j < Dv; ++j) {
            double acc = 0.0;
            for (long c = 0; c < Dk; ++c) acc += S[c * Dv + j] * (scale * qt[c]);
            ot[j] = acc;
        }
#endif
        /* 4. write: H = H~ + k e^T */
        for (long c = 0; c < Dk; ++c)
            for (long j = 0; j < Dv; ++j) {
#if KDA_MUTANT == 6
                S[c * Dv + j] += kt[j % Dk] * e[c % Dv];   /* mutant: transposed outer product */
#else
                S[c * Dv + j] += kt[c] * e[j];
#endif
            }

#if KDA_MUTANT != 5
        /* 5. read: o = H^T (scale q) */
        for (long j = 0; j < Dv; ++j) {
            double acc = 0.0;
            for (long c = 0; c < Dk; ++c) {
#if KDA_MUTANT == 7
                acc += S[c * Dv + j] * qt[c];          /* mutant: scale dropped */
#else
                acc += S[c * Dv + j] * (scale * qt[c]);
#endif
            }
            ot[j] = acc;
        }
#endif
#if KDA_MUTANT == 8
        /* mutant: the gate of step t applied a second time after the write */
        if (mode == ORACLE_CHANNEL) {
            for (long c = 0; c < Dk; ++c) {
                const double a = exp(g[tok * Dk + c]);
                for (long j = 0; j < Dv; ++j) S[c * Dv + j] *= a;
            }
        } else if (mode == ORACLE_SCALAR) {
            const double a = exp(g[tok]);
            for (long i = 0; i < Dk * Dv; ++i) S[i] *= a;
        }
#endif
    }
    if (hT)
        memcpy(hT + (b * H + h) * Dk * Dv, S, sizeof(double) * Dk * Dv);
}

int kda_oracle_recurrent(const double* q, const double* k, const double* v,
                         const double* g, const double* beta, const double* h0,
                         double* o, double* hT,
                         long B, long T, long H, long Dk, long Dv,
                         double scale, int mode, int nthreads)
{
    if (!q || !k || !v || !beta || !o || B < 0 || T < 0 || H < 0 || Dk <= 0 || Dv <= 0)
        return -1;
    if (mode != ORACLE_CHANNEL && mode != ORACLE_SCALAR && mode != ORACLE_NONE)
        return -1;
    if (mode != ORACLE_NONE && !g)
        return -1;
    const long units = B * H;
    int failed = 0;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel num_threads(nthreads) reduction(| : failed)
#endif
    {
        double* S = (double*)malloc(sizeof(double) * (Dk * Dv + 2 * Dv));
        if (!S) failed = 1;
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
        for (long u = 0; u < units; ++u) {
            if (!S) continue;
            one_sequence(q, k, v, g, beta, h0, o, hT, u / H, u % H, T, H, Dk, Dv,
                         scale, mode, S, S + Dk * Dv, S + Dk * Dv + Dv);
        }
        free(S);
    }
    return failed ? -2 : 0;
}

int kda_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
