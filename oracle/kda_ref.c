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

/*
 * Gradient of the recurrence (reverse mode), fp64.
 *
 * For a scalar loss L with given dL/do_t (dO) and dL/dS_T (dS_T, NULL => 0),
 * returns dL/dq, dL/dk, dL/dv, dL/dg, dL/dbeta and dL/dS0.  This is the chain
 * rule applied to the five lines of one step of the loop in one_head(), taken
 * in reverse order; with S' = Diag(e^{g_t}) S_{t-1}, r = S'^T k_t,
 * u = beta_t (v_t - r), S_t = S' + k_t u^T, o_t = S_t^T q_t and D = dL/dS_t:
 *
 *     D     += q_t do_t^T                 dq_t  = S_t do_t
 *     du     = D^T k_t                    dk_t  = D u
 *     dbeta_t = du . (v_t - r)            dv_t  = beta_t du
 *     dr     = -beta_t du                 dk_t += S' dr,   D += k_t dr^T
 *     dg_t[c] = sum_j D[c,j] S'[c,j]      dL/dS_{t-1} = Diag(e^{g_t}) D
 *
 * The backward sweep needs S_{t-1} for every t.  The forward pass keeps the
 * state at every SEG-th token; each segment's states are then recomputed from
 * its checkpoint with the same arithmetic as the forward pass, so they are the
 * forward states bit for bit.
 */
#define SEG 64

static void fwd_step(double* S, const double* kt, const double* gt, const double* vt,
                     double bt, long dk, long dv, double* r)
{
    for (long c = 0; c < dk; ++c) {
        const double a = exp(gt[c]);
        double* row = S + c * dv;
        for (long j = 0; j < dv; ++j) row[j] *= a;
    }
    for (long j = 0; j < dv; ++j) r[j] = 0.0;
    for (long c = 0; c < dk; ++c) {
        const double* row = S + c * dv;
        for (long j = 0; j < dv; ++j) r[j] += row[j] * kt[c];
    }
    for (long j = 0; j < dv; ++j) r[j] = bt * (vt[j] - r[j]);
    for (long c = 0; c < dk; ++c) {
        double* row = S + c * dv;
        for (long j = 0; j < dv; ++j) row[j] += kt[c] * r[j];
    }
}

static int one_head_grad(const double* q, const double* k, const double* v,
                         const double* g, const double* beta, const double* S0,
                         const double* dO, const double* dST,
                         double* dq, double* dk_, double* dv_, double* dg, double* dbeta,
                         double* dS0, long T, long H, long dk, long dv)
{
    const long sk = H * dk, sv = H * dv, DD = dk * dv;
    const long nseg = (T + SEG - 1) / SEG;
    double* ck = (double*)malloc(sizeof(double) * (size_t)((nseg > 0 ? nseg : 1) * DD));
    double* seg = (double*)malloc(sizeof(double) * (size_t)((SEG + 1) * DD));
    double* Sp = (double*)malloc(sizeof(double) * (size_t)DD);
    double* D = (double*)malloc(sizeof(double) * (size_t)DD);
    double* r = (double*)malloc(sizeof(double) * (size_t)dv);
    double* u = (double*)malloc(sizeof(double) * (size_t)dv);
    double* du = (double*)malloc(sizeof(double) * (size_t)dv);
    if (!ck || !seg || !Sp || !D || !r || !u || !du) {
        free(ck); free(seg); free(Sp); free(D); free(r); free(u); free(du);
        return -1;
    }

    /* forward pass: checkpoint the state entering every segment */
    double* S = seg;
    if (S0) memcpy(S, S0, sizeof(double) * DD);
    else memset(S, 0, sizeof(double) * DD);
    for (long t = 0; t < T; ++t) {
        if (t % SEG == 0) memcpy(ck + (t / SEG) * DD, S, sizeof(double) * DD);
        fwd_step(S, k + t * sk, g + t * sk, v + t * sv, beta[t * H], dk, dv, r);
    }

    /* backward sweep */
    if (dST) memcpy(D, dST, sizeof(double) * DD);
    else memset(D, 0, sizeof(double) * DD);
    for (long s = nseg - 1; s >= 0; --s) {
        const long t0 = s * SEG, t1 = (t0 + SEG < T) ? t0 + SEG : T;
        /* seg[i] = S_{t0 + i - 1}, i.e. the state before token t0 + i */
        memcpy(seg, ck + s * DD, sizeof(double) * DD);
        for (long t = t0; t < t1 - 1; ++t) {
            double* nxt = seg + (t - t0 + 1) * DD;
            memcpy(nxt, seg + (t - t0) * DD, sizeof(double) * DD);
            fwd_step(nxt, k + t * sk, g + t * sk, v + t * sv, beta[t * H], dk, dv, r);
        }
        for (long t = t1 - 1; t >= t0; --t) {
            const double* qt = q + t * sk;
            const double* kt = k + t * sk;
            const double* gt = g + t * sk;
            const double* vt = v + t * sv;
            const double* dot = dO + t * sv;
            const double bt = beta[t * H];
            const double* Sprev = seg + (t - t0) * DD;

            /* recompute S', r, u and S_t (S_t into the buffer after Sprev) */
            for (long c = 0; c < dk; ++c) {
                const double a = exp(gt[c]);
                for (long j = 0; j < dv; ++j) Sp[c * dv + j] = a * Sprev[c * dv + j];
            }
            for (long j = 0; j < dv; ++j) r[j] = 0.0;
            for (long c = 0; c < dk; ++c)
                for (long j = 0; j < dv; ++j) r[j] += Sp[c * dv + j] * kt[c];
            for (long j = 0; j < dv; ++j) u[j] = bt * (vt[j] - r[j]);

            /* o_t = S_t^T q_t  with  S_t = S' + k_t u^T */
            double* dqt = dq + t * sk;
            for (long c = 0; c < dk; ++c) {
                double acc = 0.0;
                for (long j = 0; j < dv; ++j) acc += (Sp[c * dv + j] + kt[c] * u[j]) * dot[j];
                dqt[c] = acc;
            }
            for (long c = 0; c < dk; ++c)
                for (long j = 0; j < dv; ++j) D[c * dv + j] += qt[c] * dot[j];

            /* S_t = S' + k_t u^T */
            double* dkt = dk_ + t * sk;
            for (long j = 0; j < dv; ++j) du[j] = 0.0;
            for (long c = 0; c < dk; ++c) {
                double acc = 0.0;
                for (long j = 0; j < dv; ++j) {
                    du[j] += D[c * dv + j] * kt[c];
                    acc += D[c * dv + j] * u[j];
                }
                dkt[c] = acc;
            }

            /* u = beta_t (v_t - r) */
            double db = 0.0;
            double* dvt = dv_ + t * sv;
            for (long j = 0; j < dv; ++j) {
                db += du[j] * (vt[j] - r[j]);
                dvt[j] = bt * du[j];
                du[j] = -bt * du[j];           /* now dL/dr */
            }
            dbeta[t * H] = db;

            /* r = S'^T k_t */
            for (long c = 0; c < dk; ++c) {
                double acc = 0.0;
                for (long j = 0; j < dv; ++j) {
                    acc += Sp[c * dv + j] * du[j];
                    D[c * dv + j] += kt[c] * du[j];
                }
                dkt[c] += acc;
            }

            /* S' = Diag(e^{g_t}) S_{t-1} */
            double* dgt = dg + t * sk;
            for (long c = 0; c < dk; ++c) {
                const double a = exp(gt[c]);
                double acc = 0.0;
                for (long j = 0; j < dv; ++j) {
                    acc += D[c * dv + j] * Sp[c * dv + j];
                    D[c * dv + j] *= a;
                }
                dgt[c] = acc;
            }
        }
    }
    if (dS0) memcpy(dS0, D, sizeof(double) * DD);
    free(ck); free(seg); free(Sp); free(D); free(r); free(u); free(du);
    return 0;
}

/* Gradient of the recurrence for every (batch, head).  Layouts as for
 * kda_ref_recurrent; dO has the layout of o, dS_T and dS0 that of S0.  S0,
 * dS_T and dS0 may be NULL.  Returns 0 on success, -1 on bad arguments or
 * allocation failure. */
int kda_ref_recurrent_grad(const double* q, const double* k, const double* v,
                           const double* g, const double* beta, const double* S0,
                           const double* dO, const double* dS_T,
                           double* dq, double* dk_, double* dv_, double* dg, double* dbeta,
                           double* dS0, long B, long T, long H, long dk, long dv,
                           int nthreads)
{
    if (!q || !k || !v || !g || !beta || !dO || !dq || !dk_ || !dv_ || !dg || !dbeta) return -1;
    if (B < 0 || T < 0 || H < 0 || dk <= 0 || dv <= 0) return -1;
    const long pairs = B * H;
    int err = 0;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads) reduction(|:err)
#endif
    for (long p = 0; p < pairs; ++p) {
        const long b = p / H, h = p % H;
        const long tok0 = b * T * H + h;
        err |= one_head_grad(q + tok0 * dk, k + tok0 * dk, v + tok0 * dv, g + tok0 * dk,
                             beta + tok0, S0 ? S0 + p * dk * dv : NULL, dO + tok0 * dv,
                             dS_T ? dS_T + p * dk * dv : NULL,
                             dq + tok0 * dk, dk_ + tok0 * dk, dv_ + tok0 * dv, dg + tok0 * dk,
                             dbeta + tok0, dS0 ? dS0 + p * dk * dv : NULL, T, H, dk, dv) ? 1 : 0;
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
