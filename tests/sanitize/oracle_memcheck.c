/* Host-only driver for the fp64 oracle, built with AddressSanitizer and UndefinedBehaviorSanitizer
 * together with oracle/oracle.c. Every array is allocated at exactly the size the oracle's
 * documented layout gives, so any read or write past an extent aborts the run. It covers ragged
 * shapes, the optional inputs absent and present, both input gains, every thread count path, and the
 * rejection of invalid arguments; results must be bitwise identical for every thread count. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_scan_fwd(const double *u, const double *delta, const double *A, const double *B, const double *C,
                    const double *D, const double *z, const double *delta_bias, int softplus_flag, int zoh_flag,
                    int64_t nb, int64_t nd, int64_t L, int64_t N, double *out, double *last_state, int nthreads);
int oracle_state_update(double *state, const double *x, const double *delta, const double *A, const double *B,
                        const double *C, const double *D, const double *z, int zoh_flag, int64_t nb, int64_t nd,
                        int64_t N, double *out);
int oracle_causal_conv1d(const double *x, const double *w, const double *bias, int silu_flag, int64_t nb,
                         int64_t nd, int64_t L, int64_t K, double *out);
int oracle_conv_window_update(double *window, const double *x, const double *w, const double *bias, int silu_flag,
                              int64_t nb, int64_t nd, int64_t K, double *out);
int oracle_scan_bwd(const double *u, const double *delta, const double *A, const double *B, const double *C,
                    const double *D, const double *z, const double *delta_bias, int softplus_flag, const double *dout,
                    int64_t nb, int64_t nd, int64_t L, int64_t N, double *du, double *ddelta, double *dA, double *dB,
                    double *dC, double *dD, double *dz, double *ddelta_bias);

static int failures = 0;
static uint64_t lcg = 0x9E3779B97F4A7C15ull;

/* A uniform value in [lo, hi) from a 64-bit linear congruential generator (Knuth's MMIX constants). */
static double uni(double lo, double hi) {
    lcg = lcg * 6364136223846793005ull + 1442695040888963407ull;
    return lo + (hi - lo) * (double)(lcg >> 11) * (1.0 / 9007199254740992.0);
}

static double *arr(int64_t n, double lo, double hi) {
    double *p = (double *)malloc((size_t)n * sizeof(double));
    for (int64_t i = 0; i < n; ++i) p[i] = uni(lo, hi);
    return p;
}

static void check(int cond, const char *what) {
    if (!cond) {
        printf("FAIL %s\n", what);
        ++failures;
    }
}

static void scan_case(int64_t nb, int64_t nd, int64_t L, int64_t N, int optional, int zoh) {
    double *u = arr(nb * nd * L, -1, 1), *dl = arr(nb * nd * L, -1, 1), *A = arr(nd * N, -2, -0.1);
    double *B = arr(nb * L * N, -1, 1), *C = arr(nb * L * N, -1, 1);
    double *D = optional ? arr(nd, 0.5, 1.5) : NULL, *z = optional ? arr(nb * nd * L, -2, 2) : NULL;
    double *bias = optional ? arr(nd, -3, 0) : NULL;
    double *o1 = arr(nb * nd * L, 0, 0), *o2 = arr(nb * nd * L, 0, 0), *o3 = arr(nb * nd * L, 0, 0);
    double *s1 = arr(nb * nd * N, 0, 0), *s2 = arr(nb * nd * N, 0, 0);
    check(oracle_scan_fwd(u, dl, A, B, C, D, z, bias, 1, zoh, nb, nd, L, N, o1, s1, 1) == 0, "scan 1 thread");
    check(oracle_scan_fwd(u, dl, A, B, C, D, z, bias, 1, zoh, nb, nd, L, N, o2, s2, 3) == 0, "scan 3 threads");
    check(oracle_scan_fwd(u, dl, A, B, C, D, z, bias, 1, zoh, nb, nd, L, N, o3, NULL, 0) == 0, "scan all cores");
    check(memcmp(o1, o2, (size_t)(nb * nd * L) * sizeof(double)) == 0, "scan out thread-count invariant");
    check(memcmp(o1, o3, (size_t)(nb * nd * L) * sizeof(double)) == 0, "scan out without last_state");
    check(memcmp(s1, s2, (size_t)(nb * nd * N) * sizeof(double)) == 0, "scan state thread-count invariant");
    /* the backward on the same inputs (Euler gain only) */
    if (!zoh) {
        double *dout = arr(nb * nd * L, -1, 1);
        double *du = arr(nb * nd * L, 0, 0), *dd = arr(nb * nd * L, 0, 0), *dA = arr(nd * N, 0, 0);
        double *dB = arr(nb * L * N, 0, 0), *dC = arr(nb * L * N, 0, 0), *dD = arr(nd, 0, 0);
        double *dz = arr(nb * nd * L, 0, 0), *db = arr(nd, 0, 0);
        check(oracle_scan_bwd(u, dl, A, B, C, D, z, bias, 1, dout, nb, nd, L, N, du, dd, dA, dB, dC, dD,
                              optional ? dz : NULL, db) == 0, "bwd");
        check(oracle_scan_bwd(u, dl, A, B, C, D, z, bias, 0, dout, nb, nd, L, N, du, dd, dA, dB, dC, NULL,
                              optional ? dz : NULL, NULL) == 0, "bwd softplus off, sums omitted");
        free(dout); free(du); free(dd); free(dA); free(dB); free(dC); free(dD); free(dz); free(db);
    }
    /* decode steps over the same sequence */
    double *st = arr(nb * nd * N, 0, 0), *x = malloc((size_t)(nb * nd) * sizeof(double));
    double *d1 = malloc((size_t)(nb * nd) * sizeof(double)), *zt = malloc((size_t)(nb * nd) * sizeof(double));
    double *Bt = malloc((size_t)(nb * N) * sizeof(double)), *Ct = malloc((size_t)(nb * N) * sizeof(double));
    double *out = malloc((size_t)(nb * nd) * sizeof(double));
    for (int64_t t = 0; t < L; ++t) {
        for (int64_t r = 0; r < nb * nd; ++r) {
            x[r] = u[r * L + t];
            d1[r] = dl[r * L + t];
            zt[r] = z ? z[r * L + t] : 0.0;
        }
        for (int64_t b = 0; b < nb; ++b)
            for (int64_t n = 0; n < N; ++n) {
                Bt[b * N + n] = B[(b * L + t) * N + n];
                Ct[b * N + n] = C[(b * L + t) * N + n];
            }
        check(oracle_state_update(st, x, d1, A, Bt, Ct, D, z ? zt : NULL, zoh, nb, nd, N, out) == 0, "update");
    }
    free(st); free(x); free(d1); free(zt); free(Bt); free(Ct); free(out);
    free(u); free(dl); free(A); free(B); free(C); free(D); free(z); free(bias);
    free(o1); free(o2); free(o3); free(s1); free(s2);
}

static void conv_case(int64_t nb, int64_t nd, int64_t L, int64_t K, int with_bias) {
    double *x = arr(nb * nd * L, -1, 1), *w = arr(nd * K, -1, 1), *b = with_bias ? arr(nd, -1, 1) : NULL;
    double *out = arr(nb * nd * L, 0, 0), *win = arr(nb * nd * K, 0, 0);
    double *xt = malloc((size_t)(nb * nd) * sizeof(double)), *ot = malloc((size_t)(nb * nd) * sizeof(double));
    check(oracle_causal_conv1d(x, w, b, 1, nb, nd, L, K, out) == 0, "conv");
    for (int64_t t = 0; t < L; ++t) {
        for (int64_t r = 0; r < nb * nd; ++r) xt[r] = x[r * L + t];
        check(oracle_conv_window_update(win, xt, w, b, 1, nb, nd, K, ot) == 0, "window");
        for (int64_t r = 0; r < nb * nd; ++r) check(ot[r] == out[r * L + t], "window step equals the sequence");
    }
    free(x); free(w); free(b); free(out); free(win); free(xt); free(ot);
}

int main(void) {
    const int64_t shapes[][4] = {{1, 1, 1, 1}, {2, 3, 7, 5}, {1, 5, 33, 16}, {3, 2, 4, 16}, {1, 64, 17, 3}};
    for (unsigned i = 0; i < sizeof(shapes) / sizeof(shapes[0]); ++i)
        for (int opt = 0; opt < 2; ++opt)
            for (int zoh = 0; zoh < 2; ++zoh) scan_case(shapes[i][0], shapes[i][1], shapes[i][2], shapes[i][3], opt, zoh);
    const int64_t cshapes[][4] = {{1, 1, 1, 1}, {2, 3, 9, 4}, {1, 4, 3, 8}, {2, 2, 5, 2}};
    for (unsigned i = 0; i < sizeof(cshapes) / sizeof(cshapes[0]); ++i)
        for (int bias = 0; bias < 2; ++bias) conv_case(cshapes[i][0], cshapes[i][1], cshapes[i][2], cshapes[i][3], bias);
    /* invalid arguments are rejected without touching memory */
    double one = 1.0;
    check(oracle_scan_fwd(NULL, &one, &one, &one, &one, NULL, NULL, NULL, 1, 0, 1, 1, 1, 1, &one, NULL, 1) != 0,
          "scan null");
    check(oracle_scan_fwd(&one, &one, &one, &one, &one, NULL, NULL, NULL, 1, 0, 0, 1, 1, 1, &one, NULL, 1) != 0,
          "scan empty");
    check(oracle_state_update(&one, &one, &one, &one, &one, &one, NULL, NULL, 0, 1, -1, 1, &one) != 0, "update shape");
    check(oracle_causal_conv1d(&one, &one, NULL, 1, 1, 1, 1, 0, &one) != 0, "conv width 0");
    check(oracle_conv_window_update(NULL, &one, &one, NULL, 1, 1, 1, 1, &one) != 0, "window null");
    check(oracle_scan_bwd(&one, &one, &one, &one, &one, NULL, NULL, NULL, 1, &one, 1, 1, 0, 1, &one, &one, &one, &one,
                          &one, NULL, NULL, NULL) != 0, "bwd empty");
    if (failures) {
        printf("%d failures\n", failures);
        return 1;
    }
    printf("oracle memcheck ok\n");
    return 0;
}
