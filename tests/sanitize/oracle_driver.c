/*
 * Drives every function of oracle/rsu_oracle.c on small random heads (d_k = 8, d_v = 6),
 * for a build with the host address and undefined-behaviour sanitizers: any out-of-bounds
 * access, use after free, leak or undefined operation ends the run with an error. Exits 0
 * when every output is finite.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

void oracle_dense_step(int64_t, int, int, int, double *, const double *, const double *, const double *,
                       const double *, const double *, double *);
void oracle_rwkv6_step(int64_t, int, int, double *, const double *, const double *, const double *,
                       const double *, double *);
void oracle_rwkv7_step(int64_t, int, int, double *, const double *, const double *, const double *,
                       const double *, const double *, const double *, double *);
void oracle_deltaproduct_step(int64_t, int, int, int, double *, const double *, const double *,
                              const double *, const double *, const double *, double *);
void oracle_q8_quantize(int64_t, int, const double *, int8_t *, float *, double *);
void oracle_q8_window_step(int64_t, int, int, int, int, int, int8_t *, float *, double *, double *, double *,
                           const double *, const double *, const double *, const double *, const double *,
                           double *, double *, double *);
void oracle_rwkv7_q8_window_step(int64_t, int, int, int, int, int8_t *, float *, double *, double *, double *,
                                 const double *, const double *, const double *, const double *,
                                 const double *, const double *, double *, double *, double *);
void oracle_deltaproduct_q8_window_step(int64_t, int, int, int, int, int, int8_t *, float *, double *,
                                        double *, double *, const double *, const double *, const double *,
                                        const double *, const double *, double *, double *, double *);
void oracle_log_step(int64_t, int, int, int, int, int, double *, double *, double *, double *, double *,
                     const double *, const double *, const double *, const double *, const double *, double *);
void oracle_log_step_slots(int64_t, int, int, int, int, int *, double *, double *, double *, double *, double *,
                           const double *, const double *, const double *, const double *, const double *,
                           double *);
void oracle_rwkv6_log_step(int64_t, int, int, int, int, double *, double *, double *, double *, double *,
                           const double *, const double *, const double *, const double *, double *);
void oracle_rwkv6_log_step_slots(int64_t, int, int, int, int *, double *, double *, double *, double *,
                                 double *, const double *, const double *, const double *, const double *,
                                 double *);

static uint64_t state = 88172645463325252ull;
static double urand(void) { /* xorshift64 in [0, 1) */
    state ^= state << 13;
    state ^= state >> 7;
    state ^= state << 17;
    return (double)(state >> 11) / 9007199254740992.0;
}
static double *vec(size_t n, double lo, double hi) {
    double *x = (double *)malloc(sizeof(double) * n);
    for (size_t i = 0; i < n; ++i) x[i] = lo + (hi - lo) * urand();
    return x;
}
static int bad = 0;
static void finite(const char *what, const double *x, size_t n) {
    for (size_t i = 0; i < n; ++i)
        if (!isfinite(x[i])) {
            fprintf(stderr, "%s: element %zu is not finite\n", what, i);
            bad = 1;
            return;
        }
}

int main(void) {
    const int64_t nh = 3;
    const int dk = 8, dv = 6, W = 3, n = 2, C = 3;
    double *S = vec(nh * dk * dv, -0.1, 0.1), *q = vec(nh * dk, -1, 1), *k = vec(nh * n * dk, -0.5, 0.5);
    double *v = vec(nh * n * dv, -1, 1), *g = vec(nh * dk, 0.8, 1.0), *b = vec(nh * n, 0, 1);
    double *kap = vec(nh * dk, -0.5, 0.5), *a = vec(nh * dk, 0, 1), *y = vec(nh * dv, 0, 0);

    oracle_dense_step(nh, dk, dv, 0, S, q, k, v, g, b, y);
    oracle_dense_step(nh, dk, dv, 1, S, q, k, v, g, b, y);
    oracle_rwkv6_step(nh, dk, dv, S, q, k, v, g, y);
    oracle_rwkv7_step(nh, dk, dv, S, q, k, v, g, kap, a, y);
    oracle_deltaproduct_step(nh, dk, dv, n, S, q, k, v, g, b, y);
    finite("dense steps", S, nh * dk * dv);

    int8_t *Z = (int8_t *)malloc(nh * dk * dv);
    float *az = (float *)malloc(sizeof(float) * nh * dk);
    double *wz = vec(nh * dk * dv, 0, 0), *Sw = vec(nh * dk * dv, 0, 0);
    oracle_q8_quantize(nh * dk, dv, S, Z, az, wz);
    for (int per_key = 0; per_key < 2; ++per_key) {
        double *G = vec(nh * W * dk, 0, 0), *K = vec(nh * W * dk, 0, 0), *U = vec(nh * W * dv, 0, 0);
        for (int pos = 0; pos < W; ++pos)
            oracle_q8_window_step(nh, dk, dv, per_key, W, pos, Z, az, G, K, U, q, k, v, g, b, y, Sw, wz);
        finite("q8 window", y, nh * dv);
        free(G); free(K); free(U);
    }
    {
        double *G = vec(nh * 2 * W * dk, 0, 0), *K = vec(nh * 2 * W * dk, 0, 0), *U = vec(nh * 2 * W * dv, 0, 0);
        for (int pos = 0; pos < W; ++pos)
            oracle_rwkv7_q8_window_step(nh, dk, dv, W, pos, Z, az, G, K, U, q, k, v, g, kap, a, y, Sw, wz);
        finite("rwkv7 q8 window", y, nh * dv);
        free(G); free(K); free(U);
    }
    {
        double *G = vec(nh * n * W, 0, 0), *K = vec(nh * n * W * dk, 0, 0), *U = vec(nh * n * W * dv, 0, 0);
        for (int pos = 0; pos < W; ++pos)
            oracle_deltaproduct_q8_window_step(nh, dk, dv, n, W, pos, Z, az, G, K, U, q, k, v, g, b, y, Sw, wz);
        finite("deltaproduct q8 window", y, nh * dv);
        free(G); free(K); free(U);
    }
    for (int per_key = 0; per_key < 2; ++per_key) {
        double *Sb = vec(nh * dk * dv, -0.1, 0.1), *lb = vec(nh * dk, 0, 0);
        double *K = vec(nh * C * dk, 0, 0), *U = vec(nh * C * dv, 0, 0), *Lm = vec(nh * C * dk, 0, 0);
        for (int t = 0; t <= C; ++t)
            oracle_log_step(nh, dk, dv, per_key, C, t, Sb, lb, K, U, Lm, q, k, v, g, b, y);
        int Ls[3] = {0, 1, 3};
        for (int t = 0; t < 5; ++t) {
            oracle_log_step_slots(nh, dk, dv, per_key, C, Ls, Sb, lb, K, U, Lm, q, k, v, g, b, y);
            for (int i = 0; i < 3; ++i) Ls[i] = Ls[i] < C ? Ls[i] + 1 : 0;
        }
        finite("log", Sb, nh * dk * dv);
        free(Sb); free(lb); free(K); free(U); free(Lm);
    }
    {
        double *Sb = vec(nh * dk * dv, -0.1, 0.1), *lb = vec(nh * dk, 0, 0);
        double *K = vec(nh * C * dk, 0, 0), *U = vec(nh * C * dv, 0, 0), *Lm = vec(nh * C * dk, 0, 0);
        for (int t = 0; t <= C; ++t) oracle_rwkv6_log_step(nh, dk, dv, C, t, Sb, lb, K, U, Lm, q, k, v, g, y);
        int Ls[3] = {2, 0, 3};
        for (int t = 0; t < 5; ++t) {
            oracle_rwkv6_log_step_slots(nh, dk, dv, C, Ls, Sb, lb, K, U, Lm, q, k, v, g, y);
            for (int i = 0; i < 3; ++i) Ls[i] = Ls[i] < C ? Ls[i] + 1 : 0;
        }
        finite("rwkv6 log", Sb, nh * dk * dv);
        free(Sb); free(lb); free(K); free(U); free(Lm);
    }
    free(S); free(q); free(k); free(v); free(g); free(b); free(kap); free(a); free(y);
    free(Z); free(az); free(wz); free(Sw);
    if (!bad) printf("oracle driver ok\n");
    return bad;
}
