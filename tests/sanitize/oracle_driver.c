/*
 * oracle_driver.c -- runs the C oracle (oracle/gdn_serial.c) under
 * AddressSanitizer and UBSan on small shapes that reach every indexing path:
 * GQA groups, Dk != Dv, one token, a long ragged sequence, several threads,
 * the gated entries (float and double inputs) and the gate and norm helpers,
 * plus its shape-error returns. Any out-of-bounds access or undefined
 * behaviour aborts the run; the outputs are checked to be finite and, for a
 * split sequence, equal to the one-call result.
 */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_gdn_serial(const float* q, const float* k, const float* v, const float* g_log,
                      const float* beta, double scale, double* state, double* out, long B, long Hk,
                      long Hv, long S, long Dk, long Dv, int nthreads);
int oracle_gdn_serial_gated(const float* q, const float* k, const float* v, const float* a,
                            const float* b, const float* A_log, const float* dt_bias, double eps,
                            double scale, double* state, double* out, long B, long Hk, long Hv,
                            long S, long Dk, long Dv, int nthreads);
int oracle_gdn_serial_gated_f64(const double* q, const double* k, const double* v,
                                const double* a, const double* b, const double* A_log,
                                const double* dt_bias, double eps, double scale, double* state,
                                double* out, long B, long Hk, long Hv, long S, long Dk, long Dv,
                                int nthreads);
int oracle_gdn_gates(const float* a, const float* b, const float* A_log, const float* dt_bias,
                     double* g_log, double* beta, long B, long Hv, long S);
int oracle_l2norm(const float* x, double eps, double* y, long rows, long D);

static unsigned long long rng = 88172645463325252ULL;
static double urand(void) {            /* xorshift64, uniform in [-1, 1) */
    rng ^= rng << 13;
    rng ^= rng >> 7;
    rng ^= rng << 17;
    return (double)(rng >> 11) / (double)(1ULL << 52) - 1.0;
}
static float* fvec(long n, double lo, double hi) {
    float* p = malloc(sizeof(float) * (size_t)(n ? n : 1));
    for (long i = 0; i < n; ++i) p[i] = (float)(lo + (hi - lo) * 0.5 * (urand() + 1.0));
    return p;
}
static double* dvec(long n) { return calloc((size_t)(n ? n : 1), sizeof(double)); }
static int all_finite(const double* x, long n) {
    for (long i = 0; i < n; ++i)
        if (!isfinite(x[i])) return 0;
    return 1;
}

static int fails = 0;
#define CHECK(c) do { if (!(c)) { fprintf(stderr, "%s:%d: %s\n", __FILE__, __LINE__, #c); ++fails; } } while (0)

static void run_shape(long B, long Hk, long Hv, long S, long Dk, long Dv, int nthreads) {
    const long nq = B * Hk * S * Dk, nv = B * Hv * S * Dv, ng = B * Hv * S, ns = B * Hv * Dk * Dv;
    float *q = fvec(nq, -0.3, 0.3), *k = fvec(nq, -0.3, 0.3), *v = fvec(nv, -1, 1);
    float *g = fvec(ng, -1.0, -0.01), *be = fvec(ng, 0.0, 1.0);
    float *a = fvec(ng, -2, 2), *bb = fvec(ng, -2, 2), *Al = fvec(Hv, 0, 2.7), *dt = fvec(Hv, -1, 1);
    double *st = dvec(ns), *out = dvec(nv), *st2 = dvec(ns), *o1 = dvec(nv);
    for (long i = 0; i < ns; ++i) st[i] = st2[i] = 0.02 * urand();
    CHECK(oracle_gdn_serial(q, k, v, g, be, 0.25, st, out, B, Hk, Hv, S, Dk, Dv, nthreads) == 0);
    CHECK(all_finite(out, nv) && all_finite(st, ns));
    /* the same sequence in two calls, state carried (one head-batch plane at a time) */
    if (S > 1 && B == 1) {
        const long s1 = S / 3;
        float *q1 = malloc(sizeof(float) * (size_t)(Hk * s1 * Dk)), *k1 = malloc(sizeof(float) * (size_t)(Hk * s1 * Dk));
        float *v1 = malloc(sizeof(float) * (size_t)(Hv * s1 * Dv)), *g1 = malloc(sizeof(float) * (size_t)(Hv * s1));
        float *b1 = malloc(sizeof(float) * (size_t)(Hv * s1));
        for (long j = 0; j < Hk; ++j) memcpy(q1 + j * s1 * Dk, q + j * S * Dk, sizeof(float) * (size_t)(s1 * Dk));
        for (long j = 0; j < Hk; ++j) memcpy(k1 + j * s1 * Dk, k + j * S * Dk, sizeof(float) * (size_t)(s1 * Dk));
        for (long h = 0; h < Hv; ++h) {
            memcpy(v1 + h * s1 * Dv, v + h * S * Dv, sizeof(float) * (size_t)(s1 * Dv));
            memcpy(g1 + h * s1, g + h * S, sizeof(float) * (size_t)s1);
            memcpy(b1 + h * s1, be + h * S, sizeof(float) * (size_t)s1);
        }
        double* oo = dvec(Hv * s1 * Dv);
        CHECK(oracle_gdn_serial(q1, k1, v1, g1, b1, 0.25, st2, oo, 1, Hk, Hv, s1, Dk, Dv, nthreads) == 0);
        for (long h = 0; h < Hv; ++h)
            for (long i = 0; i < s1 * Dv; ++i) CHECK(oo[h * s1 * Dv + i] == out[h * S * Dv + i]);
        free(q1); free(k1); free(v1); free(g1); free(b1); free(oo);
    }
    for (long i = 0; i < ns; ++i) st[i] = 0.0;
    CHECK(oracle_gdn_serial_gated(q, k, v, a, bb, Al, dt, 1e-6, 0.25, st, out, B, Hk, Hv, S, Dk, Dv,
                                  nthreads) == 0);
    CHECK(all_finite(out, nv) && all_finite(st, ns));
    double *qd = dvec(nq), *kd = dvec(nq), *vd = dvec(nv), *ad = dvec(ng), *bd = dvec(ng);
    double *Ald = dvec(Hv), *dtd = dvec(Hv);
    for (long i = 0; i < nq; ++i) { qd[i] = q[i]; kd[i] = k[i]; }
    for (long i = 0; i < nv; ++i) vd[i] = v[i];
    for (long i = 0; i < ng; ++i) { ad[i] = a[i]; bd[i] = bb[i]; }
    for (long i = 0; i < Hv; ++i) { Ald[i] = Al[i]; dtd[i] = dt[i]; }
    for (long i = 0; i < ns; ++i) st[i] = 0.0;
    CHECK(oracle_gdn_serial_gated_f64(qd, kd, vd, ad, bd, Ald, dtd, 0.0, 0.25, st, o1, B, Hk, Hv,
                                      S, Dk, Dv, nthreads) == 0);
    CHECK(all_finite(o1, nv));
    double *gd = dvec(ng), *bed = dvec(ng), *y = dvec(nq);
    CHECK(oracle_gdn_gates(a, bb, Al, dt, gd, bed, B, Hv, S) == 0);
    CHECK(all_finite(gd, ng) && all_finite(bed, ng));
    CHECK(oracle_l2norm(q, 1e-6, y, B * Hk * S, Dk) == 0);
    CHECK(all_finite(y, nq));
    free(q); free(k); free(v); free(g); free(be); free(a); free(bb); free(Al); free(dt);
    free(st); free(out); free(st2); free(o1); free(qd); free(kd); free(vd); free(ad); free(bd);
    free(Ald); free(dtd); free(gd); free(bed); free(y);
}

int main(void) {
    run_shape(1, 2, 2, 128, 64, 64, 1);
    run_shape(2, 1, 4, 5, 16, 8, 3);       /* GQA 4, Dk != Dv */
    run_shape(1, 2, 6, 1, 8, 24, 2);       /* one token */
    run_shape(3, 3, 3, 97, 12, 20, 4);     /* ragged length, odd sizes */
    run_shape(1, 1, 2, 1000, 4, 4, 8);     /* long sequence, more threads than pairs */
    /* shape errors are returned, nothing is touched */
    double st[4] = {0}, out[4] = {0};
    float x[4] = {0};
    CHECK(oracle_gdn_serial(x, x, x, x, x, 1.0, st, out, 1, 2, 3, 1, 1, 1, 1) != 0);  /* Hv % Hk */
    CHECK(oracle_gdn_serial(x, x, x, x, x, 1.0, st, out, -1, 1, 1, 1, 1, 1, 1) != 0);
    CHECK(oracle_gdn_serial_gated(x, x, x, x, x, NULL, x, 0.0, 1.0, st, out, 1, 1, 1, 1, 1, 1, 1) != 0);
    CHECK(oracle_gdn_gates(x, x, x, x, st, out, 1, 0, 1) != 0);
    CHECK(oracle_l2norm(x, 0.0, st, 1, 0) != 0);
    printf("oracle driver: %d failures\n", fails);
    return fails ? 1 : 0;
}
