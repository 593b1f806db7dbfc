/*
 * Plain fp64 CPU oracle for the Comba mixer. TEST INFRASTRUCTURE ONLY:
 * linked by the tests, the smoke check and the benchmark's CPU-baseline leg,
 * never by the device library. It shares no source with the device path.
 *
 * Recurrence (Comba: Improving Bilinear RNNs with Closed-loop Control;
 * PaperWeekly write-up, section "Comba架构：基于闭环控制理论": a
 * scalar-plus-low-rank transition with the key as feedback, correcting the
 * value first and the output second):
 *
 *     u_t = v_t - S_{t-1} k_t
 *     S_t = alpha_t S_{t-1} + beta_t u_t k_t^T
 *     o_t = S_t (q_t - d k_t)
 *
 * S has one row per value channel (V x K, K contiguous). Each row evolves on
 * its own given (k_t, alpha_t, beta_t), so the work is split over
 * (sequence, head, block of value rows) with OpenMP. Every input is fp64;
 * callers upcast the exact values the device receives.
 *
 * Layouts: q, k [B,T,H,K]; v, o [B,T,H,V]; alpha, beta [B,T,H]; d [H];
 * s0, s_final [N,H,V,K]. cu_seqlens (int32 [N+1], B == 1) or NULL (N == B).
 * s0 may be NULL (zeros); s_final may be NULL (not written).
 * Returns 0 on success, -1 on a bad argument.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int comba_oracle_forward(const double *q, const double *k, const double *v,
                         const double *alpha, const double *beta, const double *d,
                         const double *s0, const int32_t *cu_seqlens, int32_t num_seqs,
                         int32_t B, int32_t T, int32_t H, int32_t K, int32_t V,
                         int32_t rows_per_task, double *o, double *s_final,
                         int32_t nthreads)
{
    if (!q || !k || !v || !alpha || !beta || !d || !o) return -1;
    if (B <= 0 || T < 0 || H <= 0 || K <= 0 || V <= 0) return -1;
    if (cu_seqlens && B != 1) return -1;
    const int64_t N = cu_seqlens ? num_seqs : B;
    if (N <= 0) return -1;
    if (rows_per_task <= 0 || rows_per_task > V) rows_per_task = V;
    const int64_t row_blocks = (V + rows_per_task - 1) / rows_per_task;
    const int64_t tasks = N * H * row_blocks;

#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif

    int failed = 0;
#pragma omp parallel
    {
        double *S = (double *)malloc(sizeof(double) * (size_t)rows_per_task * (size_t)K);
        double *qt = (double *)malloc(sizeof(double) * (size_t)K);
        if (!S || !qt) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t task = 0; task < tasks; ++task) {
            if (!S || !qt) continue;
            const int64_t rb = task % row_blocks;
            const int64_t h = (task / row_blocks) % H;
            const int64_t n = task / (row_blocks * H);
            const int64_t r0 = rb * rows_per_task;
            const int64_t r1 = (r0 + rows_per_task < V) ? r0 + rows_per_task : V;
            const int64_t b = cu_seqlens ? 0 : n;
            const int64_t t0 = cu_seqlens ? cu_seqlens[n] : 0;
            const int64_t t1 = cu_seqlens ? cu_seqlens[n + 1] : T;

            for (int64_t r = r0; r < r1; ++r)
                for (int64_t c = 0; c < K; ++c)
                    S[(r - r0) * K + c] = s0 ? s0[((n * H + h) * V + r) * K + c] : 0.0;

            for (int64_t t = t0; t < t1; ++t) {
                const int64_t tok = (b * T + t) * H + h;
                const double *kt = k + tok * K;
                const double *qq = q + tok * K;
                const double *vt = v + tok * V;
                const double a = alpha[tok], be = beta[tok], dh = d[h];
                for (int64_t c = 0; c < K; ++c) qt[c] = qq[c] - dh * kt[c];
                for (int64_t r = r0; r < r1; ++r) {
                    double *Sr = S + (r - r0) * K;
                    double sk = 0.0;
                    for (int64_t c = 0; c < K; ++c) sk += Sr[c] * kt[c];
                    const double u = vt[r] - sk;
                    double out = 0.0;
                    for (int64_t c = 0; c < K; ++c) {
                        Sr[c] = a * Sr[c] + be * u * kt[c];
                        out += Sr[c] * qt[c];
                    }
                    o[tok * V + r] = out;
                }
            }
            if (s_final)
                for (int64_t r = r0; r < r1; ++r)
                    memcpy(s_final + ((n * H + h) * V + r) * K, S + (r - r0) * K,
                           sizeof(double) * (size_t)K);
        }
        free(S);
        free(qt);
    }
    return failed ? -1 : 0;
}

int comba_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
