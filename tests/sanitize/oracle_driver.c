/*
 * Runs every entry point of the fp64 oracle (oracle/path_oracle.c) on small
 * deterministic inputs, edge shapes included, so that a build with
 * AddressSanitizer and UndefinedBehaviorSanitizer can check its memory
 * accesses and arithmetic.  Test infrastructure only.
 *
 * Besides running clean under the sanitizers, it checks facts that hold for
 * any input: every output is finite, row 0 of the attention is o_0 = v_0
 * (the only visible key), the last transported key is the key itself, and
 * out-of-range row or position arguments are refused.
 */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_fwd_rows(int S, int L, int d, int dv, const double *q, const double *k,
                    const double *v, const double *w, const double *beta,
                    const double *logf, double scale, int nrows, const int *rows,
                    double *o, double *lse);
int oracle_transported_keys(int S, int L, int d, const double *k, const double *w,
                            const double *beta, int t, double *out);
int oracle_bwd(int S, int L, int d, int dv, const double *q, const double *k,
               const double *v, const double *w, const double *beta, const double *logf,
               double scale, const double *dout, double *dq, double *dk, double *dvv,
               double *dw, double *dbeta, double *dlogf);
int oracle_frontend(int N, int L, int Dm, int R, int H, int d, const double *x,
                    const double *Wd, const double *Wu, const double *kc, const double *ub,
                    const double *bb, const double *uf, const double *bf, double *w,
                    double *beta, double *logf);

static unsigned long long lcg_state = 88172645463325252ULL;

static double uniform(void)      /* in [-1, 1) */
{
    lcg_state = lcg_state * 6364136223846793005ULL + 1442695040888963407ULL;
    return (double)(lcg_state >> 11) / 4503599627370496.0 - 1.0;
}

static double *fill(size_t n, double lo, double hi)
{
    double *a = malloc(sizeof(double) * (n ? n : 1));
    for (size_t i = 0; i < n; ++i) a[i] = lo + (hi - lo) * 0.5 * (uniform() + 1.0);
    return a;
}

static int failures = 0;

static void expect(int ok, const char *what)
{
    if (!ok) {
        fprintf(stderr, "FAILED: %s\n", what);
        ++failures;
    }
}

static int all_finite(const double *a, size_t n)
{
    for (size_t i = 0; i < n; ++i)
        if (!isfinite(a[i])) return 0;
    return 1;
}

static void attention_case(int S, int L, int d, int dv, int gate)
{
    const size_t n = (size_t)S * L;
    double *q = fill(n * d, -1, 1), *k = fill(n * d, -1, 1), *v = fill(n * dv, -1, 1);
    double *w = fill(n * d, -1, 1), *beta = fill(n, 0, 2);
    double *logf = gate ? fill(n, -0.5, 0) : NULL;
    int *rows = malloc(sizeof(int) * n);
    for (int s = 0; s < S; ++s)
        for (int i = 0; i < L; ++i) rows[s * L + i] = i;
    double *o = malloc(sizeof(double) * n * dv), *lse = malloc(sizeof(double) * n);
    expect(oracle_fwd_rows(S, L, d, dv, q, k, v, w, beta, logf, 0.5, L, rows, o, lse) == 0,
           "fwd_rows status");
    expect(all_finite(o, n * dv) && all_finite(lse, n), "fwd_rows finite");
    for (int s = 0; s < S; ++s)
        for (int e = 0; e < dv; ++e)
            expect(fabs(o[(size_t)s * L * dv + e] - v[(size_t)s * L * dv + e]) < 1e-12,
                   "row 0 output is v_0");
    rows[0] = L;                                           /* out of range: refused */
    expect(oracle_fwd_rows(S, L, d, dv, q, k, v, w, beta, logf, 0.5, L, rows, o, lse) == -1,
           "fwd_rows range check");
    double *tk = malloc(sizeof(double) * (size_t)S * L * d);
    expect(oracle_transported_keys(S, L, d, k, w, beta, L - 1, tk) == 0, "transported status");
    expect(all_finite(tk, (size_t)S * L * d), "transported finite");
    for (int s = 0; s < S; ++s)
        for (int e = 0; e < d; ++e)
            expect(tk[((size_t)s * L + L - 1) * d + e] == k[((size_t)s * L + L - 1) * d + e],
                   "last transported key is the key itself");
    expect(oracle_transported_keys(S, L, d, k, w, beta, L, tk) == -1, "transported range check");
    expect(oracle_transported_keys(S, L, d, k, w, beta, -1, tk) == -1, "transported range check");
    double *dout = fill(n * dv, -1, 1);
    double *dq = malloc(sizeof(double) * n * d), *dk = malloc(sizeof(double) * n * d);
    double *dw = malloc(sizeof(double) * n * d), *dvv = malloc(sizeof(double) * n * dv);
    double *db = malloc(sizeof(double) * n), *dlf = gate ? malloc(sizeof(double) * n) : NULL;
    oracle_bwd(S, L, d, dv, q, k, v, w, beta, logf, 0.5, dout, dq, dk, dvv, dw, db, dlf);
    expect(all_finite(dq, n * d) && all_finite(dk, n * d) && all_finite(dw, n * d) &&
           all_finite(dvv, n * dv) && all_finite(db, n), "bwd finite");
    if (gate) expect(all_finite(dlf, n), "bwd dlogf finite");
    free(q); free(k); free(v); free(w); free(beta); free(logf); free(rows); free(o); free(lse);
    free(tk); free(dout); free(dq); free(dk); free(dw); free(dvv); free(db); free(dlf);
}

static void frontend_case(int N, int L, int Dm, int R, int H, int d, int gate)
{
    double *x = fill((size_t)N * L * Dm, -1, 1), *Wd = fill((size_t)R * Dm, -0.3, 0.3);
    double *Wu = fill((size_t)H * d * R, -0.3, 0.3), *kc = fill((size_t)H * d * 3, -1, 1);
    double *ub = fill((size_t)H * Dm, -0.3, 0.3), *bb = fill(H, -1, 1);
    double *uf = gate ? fill((size_t)H * Dm, -0.3, 0.3) : NULL, *bf = gate ? fill(H, 2, 4) : NULL;
    double *w = malloc(sizeof(double) * N * H * L * d), *beta = malloc(sizeof(double) * N * H * L);
    double *logf = gate ? malloc(sizeof(double) * N * H * L) : NULL;
    expect(oracle_frontend(N, L, Dm, R, H, d, x, Wd, Wu, kc, ub, bb, uf, bf, w, beta, logf) == 0,
           "frontend status");
    expect(all_finite(w, (size_t)N * H * L * d) && all_finite(beta, (size_t)N * H * L),
           "frontend finite");
    for (size_t i = 0; i < (size_t)N * H * L; ++i) expect(beta[i] > 0 && beta[i] < 2, "beta range");
    if (gate)
        for (size_t i = 0; i < (size_t)N * H * L; ++i) expect(logf[i] < 0, "log f negative");
    expect(oracle_frontend(0, L, Dm, R, H, d, x, Wd, Wu, kc, ub, bb, uf, bf, w, beta, logf) != 0,
           "frontend shape check");
    free(x); free(Wd); free(Wu); free(kc); free(ub); free(bb); free(uf); free(bf);
    free(w); free(beta); free(logf);
}

int main(void)
{
    attention_case(1, 1, 4, 4, 0);
    attention_case(2, 7, 4, 3, 1);
    attention_case(3, 70, 16, 16, 1);
    attention_case(1, 65, 8, 5, 0);
    frontend_case(1, 1, 16, 16, 1, 4, 1);
    frontend_case(2, 9, 32, 16, 3, 8, 0);
    frontend_case(1, 40, 48, 32, 2, 16, 1);
    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("oracle sanitizer driver: ok\n");
    return 0;
}
