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

/*
 * Reverse mode of the same recurrence, in fp64, for a loss L with
 * dL/do = do_ [B,T,H,V] and dL/dS_final = dsf [N,H,V,K] (NULL: zero).
 * Per (sequence, head), with a_t = S_{t-1} k_t, u_t = v_t - a_t,
 * S_t = alpha_t S_{t-1} + beta_t u_t k_t^T, qt_t = q_t - d k_t,
 * o_t = S_t qt_t and X the running dL/dS_t, tokens are taken backwards:
 *
 *     X     += do_t qt_t^T                 (o_t reads S_t)
 *     dqt    = S_t^T do_t   ->  dq_t = dqt, dk_t -= d dqt, dd -= dqt . k_t
 *     dalpha_t = <X, S_{t-1}>,   dbeta_t = u_t . (X k_t)
 *     du     = beta_t X k_t     ->  dv_t = du, da = -du
 *     dk_t  += beta_t X^T u_t + S_{t-1}^T da
 *     X      = alpha_t X + da k_t^T        (dL/dS_{t-1})
 *
 * and dS_0 is X after the first token. The states S_{t-1}, S_t come from a
 * forward pass: its state every 64 tokens is kept, and the states inside
 * each stretch of 64 are recomputed from it before that stretch is taken
 * backwards. One task per (sequence, head); dd_part [N,H] receives each
 * task's share of dd (the caller sums it over the sequences).
 * Outputs dq, dk [B,T,H,K], dv [B,T,H,V], dalpha, dbeta [B,T,H] are written
 * at every token of every sequence; ds0 [N,H,V,K] may be NULL.
 */
int comba_oracle_backward(const double *q, const double *k, const double *v,
                          const double *alpha, const double *beta, const double *d,
                          const double *do_, const double *s0, const double *dsf,
                          const int32_t *cu_seqlens, int32_t num_seqs,
                          int32_t B, int32_t T, int32_t H, int32_t K, int32_t V,
                          double *dq, double *dk, double *dv, double *dalpha, double *dbeta,
                          double *dd_part, double *ds0, int32_t nthreads)
{
    enum { STRETCH = 64 };
    if (!q || !k || !v || !alpha || !beta || !d || !do_) return -1;
    if (!dq || !dk || !dv || !dalpha || !dbeta || !dd_part) return -1;
    if (B <= 0 || T < 0 || H <= 0 || K <= 0 || V <= 0) return -1;
    if (cu_seqlens && B != 1) return -1;
    const int64_t N = cu_seqlens ? num_seqs : B;
    if (N <= 0) return -1;
    const int64_t VK = (int64_t)V * K;

#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif

    int failed = 0;
#pragma omp parallel
    {
        /* longest sequence bounds the checkpoint count */
        int64_t maxlen = 0;
        for (int64_t n = 0; n < N; ++n) {
            const int64_t len = cu_seqlens ? (int64_t)cu_seqlens[n + 1] - cu_seqlens[n] : T;
            if (len > maxlen) maxlen = len;
        }
        const int64_t nck = maxlen / STRETCH + 1;
        double *ck = (double *)malloc(sizeof(double) * (size_t)(nck * VK));
        double *st = (double *)malloc(sizeof(double) * (size_t)((STRETCH + 1) * VK));
        double *X = (double *)malloc(sizeof(double) * (size_t)VK);
        double *qt = (double *)malloc(sizeof(double) * (size_t)K);
        double *vec = (double *)malloc(sizeof(double) * (size_t)(2 * V + K));
        if (!ck || !st || !X || !qt || !vec) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t task = 0; task < N * H; ++task) {
            if (!ck || !st || !X || !qt || !vec) continue;
            const int64_t h = task % H, n = task / H;
            const int64_t b = cu_seqlens ? 0 : n;
            const int64_t t0 = cu_seqlens ? cu_seqlens[n] : 0;
            const int64_t t1 = cu_seqlens ? cu_seqlens[n + 1] : T;
            double *S = st;  /* working state */
            for (int64_t e = 0; e < VK; ++e) S[e] = s0 ? s0[(n * H + h) * VK + e] : 0.0;
            /* forward: keep the state before tokens t0, t0 + 64, ... */
            for (int64_t t = t0; t < t1; ++t) {
                if ((t - t0) % STRETCH == 0) memcpy(ck + ((t - t0) / STRETCH) * VK, S, sizeof(double) * (size_t)VK);
                const int64_t tok = (b * T + t) * H + h;
                const double *kt = k + tok * K;
                for (int64_t r = 0; r < V; ++r) {
                    double *Sr = S + r * K;
                    double sk = 0.0;
                    for (int64_t c = 0; c < K; ++c) sk += Sr[c] * kt[c];
                    const double u = v[tok * V + r] - sk;
                    for (int64_t c = 0; c < K; ++c) Sr[c] = alpha[tok] * Sr[c] + beta[tok] * u * kt[c];
                }
            }
            for (int64_t e = 0; e < VK; ++e) X[e] = dsf ? dsf[(n * H + h) * VK + e] : 0.0;
            double ddh = 0.0;
            const int64_t nstretch = (t1 - t0 + STRETCH - 1) / STRETCH;
            for (int64_t j = nstretch - 1; j >= 0; --j) {
                const int64_t a0 = t0 + j * STRETCH;
                const int64_t a1 = (a0 + STRETCH < t1) ? a0 + STRETCH : t1;
                /* st[i] = state before token a0 + i, i = 0 .. a1 - a0 */
                memcpy(st, ck + j * VK, sizeof(double) * (size_t)VK);
                for (int64_t t = a0; t < a1; ++t) {
                    const int64_t tok = (b * T + t) * H + h;
                    const double *kt = k + tok * K;
                    const double *Sp = st + (t - a0) * VK;
                    double *Sn = st + (t - a0 + 1) * VK;
                    for (int64_t r = 0; r < V; ++r) {
                        double sk = 0.0;
                        for (int64_t c = 0; c < K; ++c) sk += Sp[r * K + c] * kt[c];
                        const double u = v[tok * V + r] - sk;
                        for (int64_t c = 0; c < K; ++c)
                            Sn[r * K + c] = alpha[tok] * Sp[r * K + c] + beta[tok] * u * kt[c];
                    }
                }
                for (int64_t t = a1 - 1; t >= a0; --t) {
                    const int64_t tok = (b * T + t) * H + h;
                    const double *kt = k + tok * K, *qq = q + tok * K, *dot = do_ + tok * V;
                    const double *Sp = st + (t - a0) * VK, *Sc = st + (t - a0 + 1) * VK;
                    const double al = alpha[tok], be = beta[tok], dh = d[h];
                    double *ur = vec, *Xk = vec + V, *dqt = vec + 2 * V;
                    for (int64_t c = 0; c < K; ++c) qt[c] = qq[c] - dh * kt[c];
                    /* X += do_t qt^T ; dqt = S_t^T do_t */
                    for (int64_t c = 0; c < K; ++c) dqt[c] = 0.0;
                    for (int64_t r = 0; r < V; ++r)
                        for (int64_t c = 0; c < K; ++c) {
                            X[r * K + c] += dot[r] * qt[c];
                            dqt[c] += Sc[r * K + c] * dot[r];
                        }
                    double dqk = 0.0;
                    for (int64_t c = 0; c < K; ++c) {
                        dq[tok * K + c] = dqt[c];
                        dk[tok * K + c] = -dh * dqt[c];
                        dqk += dqt[c] * kt[c];
                    }
                    ddh -= dqk;
                    /* u_t = v_t - S_{t-1} k_t ; X k_t ; <X, S_{t-1}> */
                    double dal = 0.0, dbe = 0.0;
                    for (int64_t r = 0; r < V; ++r) {
                        double sk = 0.0, xk = 0.0;
                        for (int64_t c = 0; c < K; ++c) {
                            sk += Sp[r * K + c] * kt[c];
                            xk += X[r * K + c] * kt[c];
                            dal += X[r * K + c] * Sp[r * K + c];
                        }
                        ur[r] = v[tok * V + r] - sk;
                        Xk[r] = xk;
                        dbe += ur[r] * xk;
                    }
                    dalpha[tok] = dal;
                    dbeta[tok] = dbe;
                    /* du = beta X k ; dv = du ; da = -du ;
                       dk += beta X^T u + S_{t-1}^T da ; X = alpha X + da k^T */
                    for (int64_t r = 0; r < V; ++r) {
                        const double du = be * Xk[r], da = -du;
                        dv[tok * V + r] = du;
                        for (int64_t c = 0; c < K; ++c) {
                            dk[tok * K + c] += be * X[r * K + c] * ur[r] + Sp[r * K + c] * da;
                            X[r * K + c] = al * X[r * K + c] + da * kt[c];
                        }
                    }
                }
            }
            dd_part[n * H + h] = ddh;
            if (ds0) memcpy(ds0 + (n * H + h) * VK, X, sizeof(double) * (size_t)VK);
        }
        free(ck);
        free(st);
        free(X);
        free(qt);
        free(vec);
    }
    return failed ? -1 : 0;
}
