/*
 * gdn_oracle.c -- float64 CPU oracle for the gated delta rule.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, obviously correct
 * statement of what the GPU library computes.  Only the test suite, the smoke
 * check and the benchmark's CPU-baseline leg may load it; the library itself
 * never calls it and shares no code with it.
 *
 * Sources (the pages this restates):
 *   [HB7]  Handbook page "7. Gated DeltaNet: the token-by-token recurrence"
 *          (anrans.github.io/ai-infra-handbooks/en/transformer/deltanet/),
 *          and its Chinese twin "（七）Gated DeltaNet：逐 token 递推".
 *   [LLV]  learn-llm page 13_linear_attention_viz (learn-llm.fim.ai).
 *
 * What is computed, per sequence n and V head h (QK head hq = h / (HV/HQK),
 * the repeat-interleave sharing of the qwen/deltanet.py listing in [HB7]):
 *
 *   S  <- S0[n,h], or zeros                        ([HB7] delta_rule: empty table)
 *   for each token t of the sequence, in order:
 *     k^ = k / max(|k|_2, eps)                     ([HB7] "Why are q and k normalized")
 *     q^ = scale * q / max(|q|_2, eps)
 *     S  <- exp(g_t) * S                           1. decay        ([HB7] figure "one step")
 *     p  <- S^T k^                                 2. look up
 *     S  <- S + k^ (beta_t (v_t - p))^T            3. write the difference
 *     o_t <- S^T q^                                4. read
 *   S_T[n,h] <- S
 *
 * which is [HB7] "The formula":
 *   S_t = a_t S_{t-1} + b_t k_t (v_t - a_t S_{t-1}^T k_t)^T,  o_t = S_t^T q_t.
 *
 * Two switches exist for the oracle's own pins and the variant rows of the
 * [LLV] update-rule table; the method itself is delta = 1, normalize = 1:
 *   delta = 0      drop the look-up (step 2 gives p = 0): the linear-attention /
 *                  Mamba2 rows, S <- a S + b k v^T ([HB7] "The formula", the
 *                  sentence on the version without the subtraction)
 *   normalize = 0  use q and k as given ([LLV] note on |k| != 1)
 *
 * eps = 1e-12, the documented default of torch.nn.functional.normalize, which
 * [LLV] names as the normaliser; [HB7] does not show its l2norm.
 *
 * Build: cc -O2 -fopenmp -shared -fPIC gdn_oracle.c -lm   (no fast-math)
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define GDN_ORACLE_EPS 1e-12

static void unit_scaled(const double *x, double *out, int64_t d, double scale, int normalize)
{
    double r = 1.0;
    if (normalize) {
        double ss = 0.0;
        for (int64_t i = 0; i < d; ++i) ss += x[i] * x[i];
        double nrm = sqrt(ss);
        r = 1.0 / (nrm > GDN_ORACLE_EPS ? nrm : GDN_ORACLE_EPS);
    }
    for (int64_t i = 0; i < d; ++i) out[i] = scale * (x[i] * r);
}

/* One (sequence, V head) unit: the token loop above. */
static void run_unit(const double *q, const double *k, const double *v, const double *g,
                     const double *beta, int64_t t0, int64_t t1, int64_t hq, int64_t h,
                     const double *S0, double *o, double *S_T, int64_t HQK, int64_t HV,
                     int64_t dk, int64_t dv, double scale, int delta, int normalize,
                     double *S, double *kh, double *qh, double *p)
{
    if (S0) memcpy(S, S0, sizeof(double) * (size_t)(dk * dv));
    else memset(S, 0, sizeof(double) * (size_t)(dk * dv));

    for (int64_t t = t0; t < t1; ++t) {
        unit_scaled(k + (t * HQK + hq) * dk, kh, dk, 1.0, normalize);
        unit_scaled(q + (t * HQK + hq) * dk, qh, dk, scale, normalize);
        const double a = exp(g[t * HV + h]);
        const double b = beta[t * HV + h];
        const double *vt = v + (t * HV + h) * dv;

        for (int64_t i = 0; i < dk * dv; ++i) S[i] *= a;                 /* 1. decay */

        for (int64_t j = 0; j < dv; ++j) p[j] = 0.0;                      /* 2. look up */
        if (delta)
            for (int64_t i = 0; i < dk; ++i)
                for (int64_t j = 0; j < dv; ++j) p[j] += S[i * dv + j] * kh[i];

        for (int64_t j = 0; j < dv; ++j) p[j] = b * (vt[j] - p[j]);      /* 3. write */
        for (int64_t i = 0; i < dk; ++i)
            for (int64_t j = 0; j < dv; ++j) S[i * dv + j] += kh[i] * p[j];

        double *ot = o + (t * HV + h) * dv;                               /* 4. read */
        for (int64_t j = 0; j < dv; ++j) ot[j] = 0.0;
        for (int64_t i = 0; i < dk; ++i)
            for (int64_t j = 0; j < dv; ++j) ot[j] += S[i * dv + j] * qh[i];
    }
    if (S_T) memcpy(S_T, S, sizeof(double) * (size_t)(dk * dv));
}

/*
 * Packed batch.  Layouts (row-major, last index fastest):
 *   q, k [total_T, HQK, dk]; v, o [total_T, HV, dv]; g, beta [total_T, HV];
 *   cu_seqlens [n_seq + 1] (sequence n owns tokens [cu[n], cu[n+1]));
 *   S0, S_T [n_seq, HV, dk, dv] (S0 may be NULL: zeros; S_T may be NULL).
 * Returns 0, or -1 for inconsistent sizes, -2 if out of memory.
 * Runs (sequence, head) units in parallel with OpenMP when built with it.
 */
int gdn_oracle_run(const double *q, const double *k, const double *v, const double *g,
                   const double *beta, const int64_t *cu_seqlens, int64_t n_seq,
                   const double *S0, double *o, double *S_T, int64_t HQK, int64_t HV,
                   int64_t dk, int64_t dv, double scale, int delta, int normalize)
{
    if (n_seq < 0 || HQK <= 0 || HV <= 0 || dk <= 0 || dv <= 0 || HV % HQK != 0) return -1;
    for (int64_t n = 0; n < n_seq; ++n)
        if (cu_seqlens[n + 1] < cu_seqlens[n]) return -1;
    if (n_seq > 0 && cu_seqlens[0] != 0) return -1;
    const int64_t r = HV / HQK;
    const int64_t units = n_seq * HV;
    int failed = 0;

#pragma omp parallel
    {
        double *S = (double *)malloc(sizeof(double) * (size_t)(dk * dv));
        double *kh = (double *)malloc(sizeof(double) * (size_t)dk);
        double *qh = (double *)malloc(sizeof(double) * (size_t)dk);
        double *p = (double *)malloc(sizeof(double) * (size_t)dv);
        const int ok = S && kh && qh && p;
        if (!ok) {
#pragma omp atomic write
            failed = 1;
        }
        /* every thread reaches the work-sharing loop; one without buffers skips its share */
#pragma omp for schedule(dynamic, 1)
        for (int64_t u = 0; u < units; ++u) {
            if (!ok) continue;
            const int64_t n = u / HV, h = u % HV;
            const size_t off = (size_t)((n * HV + h) * dk * dv);
            run_unit(q, k, v, g, beta, cu_seqlens[n], cu_seqlens[n + 1], h / r, h,
                     S0 ? S0 + off : NULL, o, S_T ? S_T + off : NULL, HQK, HV, dk, dv,
                     scale, delta, normalize, S, kh, qh, p);
        }
        free(S); free(kh); free(qh); free(p);
    }
    return failed ? -2 : 0;
}

/* Number of threads the parallel region above would use (1 without OpenMP). */
int gdn_oracle_threads(void)
{
    int n = 1;
#pragma omp parallel
    {
#pragma omp single
        {
#ifdef _OPENMP
            n = omp_get_num_threads();
#endif
        }
    }
    return n;
}
