/* Runs the fp64 C oracle (oracle/la_oracle.c) under AddressSanitizer on exactly sized heap
 * buffers: several groups, ragged lengths, with and without a carry and an upstream gradient,
 * and the argument errors.  Every buffer is malloc'd at its exact size, so any read or write
 * past a group's slice is reported.  Also checks two closed forms that hold for any positive
 * inputs: o_1 = v_1 from a zero carry, and q_t . dq_t = 0.  Exit status 0 when all hold. */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

int la_oracle_fwd(int G, int T, int D, const double *q, const double *k, const double *v, const double *S_in,
                  const double *z_in, double *o, double *S_out, double *z_out, int nthreads);
int la_oracle_bwd(int G, int T, int D, const double *q, const double *k, const double *v, const double *S_in,
                  const double *z_in, const double *dO, const double *dS_out, const double *dz_out, double *dq,
                  double *dk, double *dv, double *dS_in, double *dz_in, int nthreads);

static unsigned long long rng = 88172645463325252ull;
static double uni(void) { /* xorshift64, uniform in [0, 1) */
    rng ^= rng << 13;
    rng ^= rng >> 7;
    rng ^= rng << 17;
    return (double)(rng >> 11) / 9007199254740992.0;
}
static double *fill(size_t n, double lo, double hi) {
    double *p = (double *)malloc(sizeof(double) * (n ? n : 1));
    for (size_t i = 0; i < n; ++i) p[i] = lo + (hi - lo) * uni();
    return p;
}

static int failures = 0;
static void check(int ok, const char *what, int G, int T, int D) {
    if (!ok) {
        printf("FAIL %s (G=%d T=%d D=%d)\n", what, G, T, D);
        ++failures;
    }
}

static void run(int G, int T, int D, int carry, int upstream, int nthreads) {
    const size_t tok = (size_t)G * T * D, st = (size_t)G * D * D, z = (size_t)G * D;
    double *q = fill(tok, 0.1, 2.0), *k = fill(tok, 0.1, 2.0), *v = fill(tok, -1.0, 1.0), *dO = fill(tok, -1, 1);
    double *S_in = carry ? fill(st, 0.0, 1.0) : NULL, *z_in = carry ? fill(z, 0.5, 2.0) : NULL;
    double *dS_out = upstream ? fill(st, -1, 1) : NULL, *dz_out = upstream ? fill(z, -1, 1) : NULL;
    double *o = fill(tok, 0, 0), *S_out = fill(st, 0, 0), *z_out = fill(z, 0, 0);
    double *dq = fill(tok, 0, 0), *dk = fill(tok, 0, 0), *dv = fill(tok, 0, 0), *dS_in = fill(st, 0, 0),
           *dz_in = fill(z, 0, 0);
    check(la_oracle_fwd(G, T, D, q, k, v, S_in, z_in, o, S_out, z_out, nthreads) == 0, "fwd status", G, T, D);
    check(la_oracle_bwd(G, T, D, q, k, v, S_in, z_in, dO, dS_out, dz_out, dq, dk, dv, dS_in, dz_in, nthreads) == 0,
          "bwd status", G, T, D);
    for (int g = 0; g < G && T > 0; ++g) {
        const double *og = o + (size_t)g * T * D, *vg = v + (size_t)g * T * D;
        if (!carry)
            for (int c = 0; c < D; ++c) check(fabs(og[c] - vg[c]) <= 1e-12 * (1 + fabs(vg[c])), "o_1 = v_1", G, T, D);
        for (int t = 0; t < T; ++t) {
            double dot = 0, scale = 0;
            for (int p = 0; p < D; ++p) {
                const size_t i = ((size_t)g * T + t) * D + p;
                dot += q[i] * dq[i];
                scale += fabs(q[i] * dq[i]);
            }
            check(fabs(dot) <= 1e-12 * (1 + scale), "q . dq = 0", G, T, D);
        }
    }
    double *all[] = {q, k, v, dO, S_in, z_in, dS_out, dz_out, o, S_out, z_out, dq, dk, dv, dS_in, dz_in};
    for (size_t i = 0; i < sizeof all / sizeof all[0]; ++i) free(all[i]);
}

int main(void) {
    run(3, 7, 4, 0, 0, 2);
    run(3, 7, 4, 1, 1, 2);
    run(2, 130, 64, 1, 0, 2);
    run(1, 1, 1, 0, 1, 1);
    run(2, 0, 8, 1, 1, 1); /* no tokens: the carry passes through */
    /* argument errors: bad sizes, half-given carries, a missing output */
    double x[4] = {1, 1, 1, 1};
    check(la_oracle_fwd(1, 1, 0, x, x, x, NULL, NULL, x, x, x, 1) == 1, "fwd D = 0", 1, 1, 0);
    check(la_oracle_fwd(1, 1, 1, x, x, x, x, NULL, x, x, x, 1) == 1, "fwd half carry", 1, 1, 1);
    check(la_oracle_bwd(1, 1, 1, x, x, x, NULL, NULL, x, x, NULL, x, x, x, x, x, 1) == 1, "bwd half upstream", 1, 1, 1);
    check(la_oracle_bwd(1, 1, 1, x, x, x, NULL, NULL, x, NULL, NULL, NULL, x, x, x, x, 1) == 1, "bwd no dq", 1, 1, 1);
    printf("%s: %d failures\n", failures ? "FAILED" : "ok", failures);
    return failures ? 1 : 0;
}
