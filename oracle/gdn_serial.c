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
 * The gated entry (oracle_gdn_serial_gated) first derives the recurrence's
 * inputs from the decode block's raw quantities ("GDN Block TKG Kernel API
 * Reference": introduction, "l2norm/beta/g" ahead of the recurrence;
 * Parameters A_log, a per-value-head log decay, and dt_bias, a per-value-head
 * bias inside a softplus), per token:
 *
 *     g_log = -exp(A_log[h]) * softplus(a[b,h,t] + dt_bias[h]),
 *             softplus(x) = ln(1 + e^x)
 *     beta  = sigmoid(b[b,h,t]) = 1 / (1 + e^{-b})
 *     k     = k_raw / sqrt(sum_i k_raw[i]^2 + eps), q likewise
 *             (q and k must be L2-normalised: "GDN CTE Kernel API
 *             Reference", Parameters query/key and Notes; the pages give no
 *             epsilon, so it is an argument)
 *
 * and then runs the same token step.
 *
 * Precision: inputs arrive as float (bf16 operands are widened exactly by the
 * caller); every product and sum is in double. The state is double in and out
 * so that chained calls (iterated decode) keep full precision.
 *
 * Layouts (row-major, contiguous):
 *   q, k  [B][Hk][S][Dk]     v, out [B][Hv][S][Dv]
 *   g_log, beta, a, b [B][Hv][S]   A_log, dt_bias [Hv]
 *   state [B][Hv][Dk][Dv]  (in/out)
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

/* ln(1 + e^x), evaluated without overflow for large x */
static double softplus(double x)
{
    return x > 0.0 ? x + log1p(exp(-x)) : log1p(exp(x));
}

static double sigmoid(double x)
{
    return 1.0 / (1.0 + exp(-x));
}

/* element i of an input array of float (f64 == 0) or double (f64 == 1) */
static double in_at(const void* p, long i, int f64)
{
    return f64 ? ((const double*)p)[i] : (double)((const float*)p)[i];
}

/* y = x / sqrt(sum x^2 + eps) over the vector x[off .. off+D-1] */
static void l2norm_row(const void* x, long off, int f64, double eps, double* y, long D)
{
    double ss = 0.0;
    for (long i = 0; i < D; ++i) ss += in_at(x, off + i, f64) * in_at(x, off + i, f64);
    const double r = 1.0 / sqrt(ss + eps);
    for (long i = 0; i < D; ++i) y[i] = in_at(x, off + i, f64) * r;
}

/* g_log and beta of token t of value head h */
static void gates(double a, double b, double A_log_h, double dt_bias_h, double* g, double* be)
{
    *g = -exp(A_log_h) * softplus(a + dt_bias_h);
    *be = sigmoid(b);
}

/*
 * One token of the recurrence on the [Dk][Dv] state St, with decay factor
 * a = e^{g}, write strength be, key kt, query qt (length Dk), value vt
 * (length Dv); u is scratch of length Dv, ot receives the output row.
 */
static void gdn_token(double* St, const double* kt, const double* qt, const double* vt,
                      double a, double be, double scale, double* u, double* ot,
                      long Dk, long Dv)
{
    /* S = a * S */
    for (long i = 0; i < Dk; ++i)
        for (long c = 0; c < Dv; ++c)
            St[i * Dv + c] *= a;

    /* u = beta * (v - S^T k) */
    for (long c = 0; c < Dv; ++c) {
        double x = 0.0;
        for (long i = 0; i < Dk; ++i) x += St[i * Dv + c] * kt[i];
        u[c] = be * (vt[c] - x);
    }

    /* S = S + k u^T */
    for (long i = 0; i < Dk; ++i)
        for (long c = 0; c < Dv; ++c)
            St[i * Dv + c] += kt[i] * u[c];

    /* o = scale * S^T q */
    for (long c = 0; c < Dv; ++c) {
        double y = 0.0;
        for (long i = 0; i < Dk; ++i) y += St[i * Dv + c] * qt[i];
        ot[c] = scale * y;
    }
}

/*
 * Every entry shares this driver. Without gates (A_log == NULL) g_log and
 * beta are the per-token decay and write strength and q, k are used as given;
 * with gates, gl/bt hold the raw a and b and q, k are normalised with eps.
 * All array inputs are float (f64 == 0) or all double (f64 == 1).
 */
static int serial(const void* q, const void* k, const void* v,
                  const void* gl, const void* bt, const void* A_log, const void* dt_bias,
                  int f64, double eps, double scale, double* state, double* out,
                  long B, long Hk, long Hv, long S, long Dk, long Dv, int nthreads)
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
        double* buf = (double*)malloc((size_t)(3 * Dk + 2 * Dv) * sizeof(double));
        if (!buf) {
#pragma omp atomic write
            failed = 1;
            continue;
        }
        double* kd = buf;
        double* qd = buf + Dk;
        double* vd = buf + 2 * Dk;
        double* u = buf + 2 * Dk + Dv;
        for (long t = 0; t < S; ++t) {
            const long kt = ((b * Hk + j) * S + t) * Dk;   /* offsets of k_t, q_t, v_t */
            const long qt = kt;
            const long vt = ((b * Hv + h) * S + t) * Dv;
            double g, be;
            if (A_log) {
                gates(in_at(gl, bh * S + t, f64), in_at(bt, bh * S + t, f64),
                      in_at(A_log, h, f64), in_at(dt_bias, h, f64), &g, &be);
                l2norm_row(k, kt, f64, eps, kd, Dk);
                l2norm_row(q, qt, f64, eps, qd, Dk);
            } else {
                g = in_at(gl, bh * S + t, f64);
                be = in_at(bt, bh * S + t, f64);
                for (long i = 0; i < Dk; ++i) {
                    kd[i] = in_at(k, kt + i, f64);
                    qd[i] = in_at(q, qt + i, f64);
                }
            }
            for (long c = 0; c < Dv; ++c) vd[c] = in_at(v, vt + c, f64);
            gdn_token(St, kd, qd, vd, exp(g), be, scale, u, out + (bh * S + t) * Dv, Dk, Dv);
        }
        free(buf);
    }
    return failed ? 2 : 0;
}

int oracle_gdn_serial(const float* q, const float* k, const float* v,
                      const float* g_log, const float* beta, double scale,
                      double* state, double* out,
                      long B, long Hk, long Hv, long S, long Dk, long Dv,
                      int nthreads)
{
    return serial(q, k, v, g_log, beta, NULL, NULL, 0, 0.0, scale, state, out,
                  B, Hk, Hv, S, Dk, Dv, nthreads);
}

int oracle_gdn_serial_gated(const float* q, const float* k, const float* v,
                            const float* a, const float* b,
                            const float* A_log, const float* dt_bias,
                            double eps, double scale, double* state, double* out,
                            long B, long Hk, long Hv, long S, long Dk, long Dv,
                            int nthreads)
{
    if (!A_log || !dt_bias) return 1;
    return serial(q, k, v, a, b, A_log, dt_bias, 0, eps, scale, state, out,
                  B, Hk, Hv, S, Dk, Dv, nthreads);
}

/* The same with every array input in double (for inputs that are themselves
 * results of other fp64 steps). */
int oracle_gdn_serial_gated_f64(const double* q, const double* k, const double* v,
                                const double* a, const double* b,
                                const double* A_log, const double* dt_bias,
                                double eps, double scale, double* state, double* out,
                                long B, long Hk, long Hv, long S, long Dk, long Dv,
                                int nthreads)
{
    if (!A_log || !dt_bias) return 1;
    return serial(q, k, v, a, b, A_log, dt_bias, 1, eps, scale, state, out,
                  B, Hk, Hv, S, Dk, Dv, nthreads);
}

/* The gates alone: g_log, beta [B][Hv][S] (double) from a, b [B][Hv][S] and
 * A_log, dt_bias [Hv]. */
int oracle_gdn_gates(const float* a, const float* b, const float* A_log, const float* dt_bias,
                     double* g_log, double* beta, long B, long Hv, long S)
{
    if (B < 0 || Hv <= 0 || S < 0) return 1;
    for (long bh = 0; bh < B * Hv; ++bh)
        for (long t = 0; t < S; ++t)
            gates((double)a[bh * S + t], (double)b[bh * S + t], (double)A_log[bh % Hv],
                  (double)dt_bias[bh % Hv], &g_log[bh * S + t], &beta[bh * S + t]);
    return 0;
}

/* The normalisation alone: y = x / sqrt(sum x^2 + eps) for each of `rows`
 * vectors of length D. */
int oracle_l2norm(const float* x, double eps, double* y, long rows, long D)
{
    if (rows < 0 || D <= 0) return 1;
    for (long r = 0; r < rows; ++r) l2norm_row(x, r * D, 0, eps, y + r * D, D);
    return 0;
}
