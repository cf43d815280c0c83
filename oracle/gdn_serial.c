/*
 * gdn_serial.c -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, token-serial fp64 reference of the gated delta rule (GDN)
 * recurrence. It is the oracle that the GPU library is checked against; only
 * the tests, the smoke entry and the bench's CPU-baseline leg may load it. It
 * shares no code, header or constant with the GPU path.
 *
 * What it computes (the recurrence the "GDN CTE Kernel API Reference" page
 * names in its introduction and Background section; the pages never print the
 * formula, the standard gated delta rule is written out here):
 *
 *   for every batch b and value head h, with key/query head j = h / (Hv/Hk)
 *   (page "GDN CTE Kernel API Reference", Notes: value head h reads key/query
 *   head h // (Hv//Hk)), starting from S = state[b,h] ([Dk][Dv], rows indexed
 *   by the key dimension, page "GDN CTE", Parameters: recurrent_state):
 *
 *     a    = exp(g_log[b,h,t])          natural-log decay factor
 *     S    = a * S                      decay first
 *     u    = beta[b,h,t] * (v_t - S^T k_t)      delta-rule correction, length Dv
 *     S    = S + k_t u^T                rank-1 write
 *     o_t  = scale * S^T q_t            read from the post-update state
 *
 *   which is S_t = e^{g_t} S_{t-1} + beta_t k_t (v_t - e^{g_t} S_{t-1}^T k_t)^T,
 *   o_t = scale S_t^T q_t.
 *
 * Precision: inputs arrive as float (bf16 operands are widened exactly by the
 * caller); every product and sum is in double. The state is double in and out
 * so that chained calls (iterated decode) keep full precision.
 *
 * Layouts (row-major, contiguous):
 *   q, k  [B][Hk][S][Dk]     v, out [B][Hv][S][Dv]
 *   g_log, beta [B][Hv][S]   state  [B][Hv][Dk][Dv]  (in/out)
 *
 * Parallelism: the (b, h) pairs are independent; they are spread over
 * nthreads OpenMP threads. Each pair runs the loop above exactly as written,
 * so the result does not depend on the thread count.
 *
 * Returns 0 on success, 1 on a shape error, 2 on allocation failure.
 */
#include <math.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int oracle_gdn_serial(const float* q, const float* k, const float* v,
                      const float* g_log, const float* beta, double scale,
                      double* state, double* out,
                      long B, long Hk, long Hv, long S, long Dk, long Dv,
                      int nthreads)
{
    if (B < 0 || Hk <= 0 || Hv <= 0 || S < 0 || Dk <= 0 || Dv <= 0) return 1;
    if (Hv % Hk != 0) return 1;
    const long G = Hv / Hk;
    int failed = 0;
    if (nthreads < 1) nthreads = 1;

#pragma omp parallel for num_threads(nthreads) schedule(dynamic, 1)
    for (long bh = 0; bh < B * Hv; ++bh) {
        const long b = bh / Hv;
        const long h = bh % Hv;
        const long j = h / G;                      /* GQA: contiguous groups */
        double* St = state + bh * Dk * Dv;         /* S[i][c] = St[i*Dv + c] */
        double* u = (double*)malloc((size_t)Dv * sizeof(double));
        if (!u) {
#pragma omp atomic write
            failed = 1;
            continue;
        }
        for (long t = 0; t < S; ++t) {
            const float* kt = k + ((b * Hk + j) * S + t) * Dk;
            const float* qt = q + ((b * Hk + j) * S + t) * Dk;
            const float* vt = v + ((b * Hv + h) * S + t) * Dv;
            const double a = exp((double)g_log[bh * S + t]);
            const double be = (double)beta[bh * S + t];
            double* ot = out + (bh * S + t) * Dv;

            /* S = a * S */
            for (long i = 0; i < Dk; ++i)
                for (long c = 0; c < Dv; ++c)
                    St[i * Dv + c] *= a;

            /* u = beta * (v - S^T k) */
            for (long c = 0; c < Dv; ++c) {
                double x = 0.0;
                for (long i = 0; i < Dk; ++i) x += St[i * Dv + c] * (double)kt[i];
                u[c] = be * ((double)vt[c] - x);
            }

            /* S = S + k u^T */
            for (long i = 0; i < Dk; ++i)
                for (long c = 0; c < Dv; ++c)
                    St[i * Dv + c] += (double)kt[i] * u[c];

            /* o = scale * S^T q */
            for (long c = 0; c < Dv; ++c) {
                double y = 0.0;
                for (long i = 0; i < Dk; ++i) y += St[i * Dv + c] * (double)qt[i];
                ot[c] = scale * y;
            }
        }
        free(u);
    }
    return failed ? 2 : 0;
}
