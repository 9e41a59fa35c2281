/*
 * kda_ref.c -- CPU oracle for Kimi Delta Attention (KDA).  TEST INFRASTRUCTURE.
 *
 * This file is the reference that the GPU library is checked against.  Only the
 * test suite, the smoke check and the CPU-baseline leg of the benchmark load it.
 * It shares no code, header, table or helper with the GPU library.
 *
 * What it computes: the plain sequential recurrence that defines KDA, in fp64,
 * one (batch, head) pair at a time (pairs are independent, so OpenMP runs them
 * in parallel).  Source: page "Kimi K3论文：Kimi Linear", section 3, eq. (1):
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *     o_t = S_t^T q_t
 *
 * with S_t a d_k x d_v matrix, alpha_t in (0,1]^{d_k} a per-channel forget gate
 * and beta_t in [0,1] a per-token write strength.  The gate is passed in log
 * space, g_t = log(alpha_t), because that is what the chunked form on page
 * "Kimi Linear：高效注意力机制在长序列处理中的创新应用", section 2.3, consumes.
 *
 * Expanding eq. (1) with S' = Diag(alpha_t) S_{t-1} gives the order of work in
 * the loop below:  S_t = S' + beta_t k_t (v_t - S'^T k_t)^T.  Nothing else is
 * reorganised: no chunking, no blocking, no fusion.
 *
 * Layouts (C order, all fp64):
 *   q, k, g : [B, T, H, dk]      v : [B, T, H, dv]      beta : [B, T, H]
 *   S0, S_T : [B, H, dk, dv]     o : [B, T, H, dv]
 * S0 may be NULL (zero initial state).  S_T may be NULL (not written).
 */
#include <stdlib.h>
#include <string.h>
#include <math.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static void one_head(const double* q, const double* k, const double* v,
                     const double* g, const double* beta, const double* S0,
                     double* o, double* S_T, long T, long H, long dk, long dv,
                     double* S, double* r)
{
    /* strides of one token in q/k/g and in v/o (the head axis sits inside) */
    const long sk = H * dk, sv = H * dv;
    if (S0) memcpy(S, S0, sizeof(double) * dk * dv);
    else memset(S, 0, sizeof(double) * dk * dv);

    for (long t = 0; t < T; ++t) {
        const double* qt = q + t * sk;
        const double* kt = k + t * sk;
        const double* gt = g + t * sk;
        const double* vt = v + t * sv;
        const double bt = beta[t * H];
        double* ot = o + t * sv;

        /* S' = Diag(alpha_t) S : row c of S scaled by alpha_t[c] = exp(g_t[c]) */
        for (long c = 0; c < dk; ++c) {
            const double a = exp(gt[c]);
            double* row = S + c * dv;
            for (long j = 0; j < dv; ++j) row[j] *= a;
        }
        /* r = S'^T k_t : what the memory currently returns for key k_t */
        for (long j = 0; j < dv; ++j) r[j] = 0.0;
        for (long c = 0; c < dk; ++c) {
            const double kc = kt[c];
            const double* row = S + c * dv;
            for (long j = 0; j < dv; ++j) r[j] += row[j] * kc;
        }
        /* delta-rule write: S = S' + beta_t k_t (v_t - r)^T */
        for (long j = 0; j < dv; ++j) r[j] = bt * (vt[j] - r[j]);
        for (long c = 0; c < dk; ++c) {
            const double kc = kt[c];
            double* row = S + c * dv;
            for (long j = 0; j < dv; ++j) row[j] += kc * r[j];
        }
        /* read-out o_t = S_t^T q_t */
        for (long j = 0; j < dv; ++j) ot[j] = 0.0;
        for (long c = 0; c < dk; ++c) {
            const double qc = qt[c];
            const double* row = S + c * dv;
            for (long j = 0; j < dv; ++j) ot[j] += row[j] * qc;
        }
    }
    if (S_T) memcpy(S_T, S, sizeof(double) * dk * dv);
}

/* Returns 0 on success, -1 on bad arguments or allocation failure. */
int kda_ref_recurrent(const double* q, const double* k, const double* v,
                      const double* g, const double* beta, const double* S0,
                      double* o, double* S_T, long B, long T, long H,
                      long dk, long dv, int nthreads)
{
    if (!q || !k || !v || !g || !beta || !o) return -1;
    if (B < 0 || T < 0 || H < 0 || dk <= 0 || dv <= 0) return -1;
    const long pairs = B * H;
    int err = 0;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads) reduction(|:err)
#endif
    for (long p = 0; p < pairs; ++p) {
        const long b = p / H, h = p % H;
        double* S = (double*)malloc(sizeof(double) * (size_t)(dk * dv));
        double* r = (double*)malloc(sizeof(double) * (size_t)dv);
        if (!S || !r) { err |= 1; free(S); free(r); continue; }
        const long tok0 = b * T * H + h; /* index of (b, t=0, h) in token units */
        one_head(q + tok0 * dk, k + tok0 * dk, v + tok0 * dv, g + tok0 * dk,
                 beta + tok0, S0 ? S0 + p * dk * dv : NULL, o + tok0 * dv,
                 S_T ? S_T + p * dk * dv : NULL, T, H, dk, dv, S, r);
        free(S);
        free(r);
    }
    (void)nthreads;
    return err ? -1 : 0;
}

/* Number of OpenMP threads the oracle would use by default (1 without OpenMP). */
int kda_ref_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
