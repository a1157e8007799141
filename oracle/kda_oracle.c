/*
 * Kimi Delta Attention (KDA) oracle: a plain fp64 CPU recurrence.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link,
 * load or call this file.  Its only users are the tests, the smoke check and
 * the CPU baseline of the benchmark.  It shares no code with the HIP library.
 *
 * What it computes (per sequence n and head h, tokens taken one at a time):
 *
 *   The nnterp Kimi-Linear page (the kimi_linear family description) defines
 *   KDA as the gated DeltaNet with one decay per key channel instead of one
 *   per head, applied to the state row by row ahead of the delta-rule update.
 *   Written out:
 *
 *     k_hat = k / sqrt(sum(k^2) + 1e-6)        (key L2 norm, eps inside the root)
 *     q_hat = scale * q / sqrt(sum(q^2) + 1e-6) (query L2 norm, then the scale)
 *     S     = diag(exp(g_t)) S                 (decay row c of S[dk,dv] by exp(g_t[c]))
 *     u     = S^T k_hat                         (what the decayed state recalls)
 *     delta = beta_t (v_t - u)
 *     S     = S + k_hat delta^T                 (delta-rule rank-1 update)
 *     o_t   = S^T q_hat                         (read after the update)
 *
 *   The L2 norm with eps inside the root and the query-only scale follow the
 *   Ascend model file, `_l2_normalize` and `_torch_chunk_kda` (q is normalised
 *   then divided by sqrt(key_dim)).  Decay-then-update-then-read is the order
 *   that file's chunk form unrolls to: its corrected keys carry the cumulative
 *   decay of the current token, and its in-chunk attention mask keeps the
 *   diagonal, so token t reads its own update.
 *
 * Inputs are float32 arrays holding the values exactly as stored (a bf16
 * tensor widened to float32 is exact).  Every value is widened to double
 * before any arithmetic.  Sequences are independent; the parallel loop runs
 * over (sequence, head) pairs and each pair is evaluated serially, so the
 * result does not depend on the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define KDA_ORACLE_OK 0
#define KDA_ORACLE_BAD_ARGS 1
#define KDA_ORACLE_NO_MEMORY 2

int kda_oracle_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads for later calls (n >= 1); the result never depends on it. */
void kda_oracle_set_threads(int n) {
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* One (sequence, head) pair, tokens [t0, t1).  S is dk*dv doubles, row-major
 * S[c*dv + j] (key channel c, value channel j).  Work vectors: qf, kf (dk),
 * u (dv). */
static void run_pair(int64_t t0, int64_t t1, int64_t h, int64_t H, int64_t dk, int64_t dv,
                     const float *q, const float *k, const float *v, const float *g,
                     const float *beta, double scale, int qk_l2norm, double *S,
                     double *qf, double *kf, double *u, double *out) {
    for (int64_t t = t0; t < t1; ++t) {
        const float *qt = q + (t * H + h) * dk;
        const float *kt = k + (t * H + h) * dk;
        const float *vt = v + (t * H + h) * dv;
        const float *gt = g + (t * H + h) * dk;
        const double b = (double)beta[t * H + h];

        double sq = 0.0, sk = 0.0;
        for (int64_t c = 0; c < dk; ++c) {
            qf[c] = (double)qt[c];
            kf[c] = (double)kt[c];
            sq += qf[c] * qf[c];
            sk += kf[c] * kf[c];
        }
        double rq = 1.0, rk = 1.0;
        if (qk_l2norm) {
            rq = 1.0 / sqrt(sq + 1e-6);
            rk = 1.0 / sqrt(sk + 1e-6);
        }
        for (int64_t c = 0; c < dk; ++c) {
            qf[c] = qf[c] * rq * scale;
            kf[c] = kf[c] * rk;
        }

        /* channel-wise decay of the state rows */
        for (int64_t c = 0; c < dk; ++c) {
            const double a = exp((double)gt[c]);
            double *row = S + c * dv;
            for (int64_t j = 0; j < dv; ++j) row[j] *= a;
        }
        /* u = S^T k_hat */
        for (int64_t j = 0; j < dv; ++j) u[j] = 0.0;
        for (int64_t c = 0; c < dk; ++c) {
            const double kc = kf[c];
            const double *row = S + c * dv;
            for (int64_t j = 0; j < dv; ++j) u[j] += kc * row[j];
        }
        /* delta = beta (v - u), stored in u */
        for (int64_t j = 0; j < dv; ++j) u[j] = b * ((double)vt[j] - u[j]);
        /* S += k_hat delta^T */
        for (int64_t c = 0; c < dk; ++c) {
            const double kc = kf[c];
            double *row = S + c * dv;
            for (int64_t j = 0; j < dv; ++j) row[j] += kc * u[j];
        }
        /* o_t = S^T q_hat */
        double *ot = out + (t * H + h) * dv;
        for (int64_t j = 0; j < dv; ++j) ot[j] = 0.0;
        for (int64_t c = 0; c < dk; ++c) {
            const double qc = qf[c];
            const double *row = S + c * dv;
            for (int64_t j = 0; j < dv; ++j) ot[j] += qc * row[j];
        }
    }
}

/*
 * Packed varlen forward.
 *   cu_seqlens      [num_seqs+1] host int64, cu[0] = 0, non-decreasing
 *   q, k            [T, H, dk] float32;  v [T, H, dv];  g [T, H, dk];  beta [T, H]
 *   initial_state   [num_seqs, H, dk, dv] float32, or NULL for zeros
 *   out             [T, H, dv] double (written)
 *   final_state     [num_seqs, H, dk, dv] double, or NULL
 * Returns 0 on success.
 */
int kda_oracle_forward(int64_t num_seqs, int64_t H, int64_t dk, int64_t dv,
                       const int64_t *cu_seqlens, const float *q, const float *k,
                       const float *v, const float *g, const float *beta,
                       const float *initial_state, double scale, int qk_l2norm,
                       double *out, double *final_state) {
    if (num_seqs < 0 || H <= 0 || dk <= 0 || dv <= 0 || !cu_seqlens) return KDA_ORACLE_BAD_ARGS;
    if (cu_seqlens[0] != 0) return KDA_ORACLE_BAD_ARGS;
    for (int64_t n = 0; n < num_seqs; ++n)
        if (cu_seqlens[n + 1] < cu_seqlens[n]) return KDA_ORACLE_BAD_ARGS;
    if (cu_seqlens[num_seqs] > 0 && (!q || !k || !v || !g || !beta || !out))
        return KDA_ORACLE_BAD_ARGS;

    int failed = 0;
    const int64_t pairs = num_seqs * H;
#pragma omp parallel
    {
        double *S = (double *)malloc(sizeof(double) * (size_t)(dk * dv));
        double *qf = (double *)malloc(sizeof(double) * (size_t)dk);
        double *kf = (double *)malloc(sizeof(double) * (size_t)dk);
        double *u = (double *)malloc(sizeof(double) * (size_t)dv);
        if (!S || !qf || !kf || !u) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t p = 0; p < pairs; ++p) {
            if (failed) continue;
            const int64_t n = p / H, h = p % H;
            const size_t state_off = (size_t)((n * H + h) * dk * dv);
            if (initial_state) {
                for (int64_t i = 0; i < dk * dv; ++i) S[i] = (double)initial_state[state_off + i];
            } else {
                memset(S, 0, sizeof(double) * (size_t)(dk * dv));
            }
            run_pair(cu_seqlens[n], cu_seqlens[n + 1], h, H, dk, dv, q, k, v, g, beta, scale,
                     qk_l2norm, S, qf, kf, u, out);
            if (final_state) memcpy(final_state + state_off, S, sizeof(double) * (size_t)(dk * dv));
        }
        free(S);
        free(qf);
        free(kf);
        free(u);
    }
    return failed ? KDA_ORACLE_NO_MEMORY : KDA_ORACLE_OK;
}
