/*
 * Reference (oracle) for causal linear attention with a carried state.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark may build, load or call this file.  It shares
 * no code, header or constant with the GPU library.
 *
 * What it computes is the plain definition, per group and in fp64, one token at
 * a time (the "cumsum" form of "Fractus-1B training optimization", section 1,
 * Bottleneck #1, and the inclusive read-after-update rule of section 2, Opt 2):
 *
 *     S_t = S_in + sum_{j<=t} k_j v_j^T      (D x D, S[p][c]: p key feature, c value feature)
 *     z_t = z_in + sum_{j<=t} k_j
 *     o_t = (S_t^T q_t) / (q_t . z_t)
 *
 * and S_out = S_T, z_out = z_T.  The backward is the reverse scan of the same
 * section (the gradient of a prefix sum is a suffix sum), written out for the
 * loss  L = sum_t <dO_t, o_t> + <dS_out, S_out> + dz_out . z_out:
 *
 *     den_t  = q_t . z_t,   dn_t = dO_t / den_t,   dden_t = -(dO_t . o_t) / den_t
 *     dq_t   = S_t dn_t + dden_t z_t
 *     Sh_t   = dS_out + sum_{i>=t} q_i dn_i^T,      zh_t = dz_out + sum_{i>=t} dden_i q_i
 *     dk_t   = Sh_t v_t + zh_t,    dv_t = Sh_t^T k_t
 *     dS_in  = Sh_1,  dz_in = zh_1
 *
 * Layout: q, k, v, o, dO, dq, dk, dv are [G][T][D]; S is [G][D][D]; z is [G][D];
 * all row-major fp64.  A NULL carry (S_in and z_in both NULL) is a zero carry;
 * a NULL dS_out/dz_out is a zero upstream gradient.
 *
 * Return value: 0 on success, 1 on bad arguments, 2 if some denominator was not
 * strictly positive (the inputs broke the positive-feature precondition).
 */
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static void set_threads(int nthreads)
{
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}

int la_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* One group's forward over T tokens.  S (D*D) and z (D) hold the carry on
 * entry and the final state on return. */
static int fwd_group(int T, int D, const double *q, const double *k, const double *v,
                     double *S, double *z, double *o)
{
    int bad = 0;
    for (int t = 0; t < T; ++t) {
        const double *qt = q + (size_t)t * D, *kt = k + (size_t)t * D, *vt = v + (size_t)t * D;
        /* update first: the state read by token t includes token t */
        for (int p = 0; p < D; ++p) {
            double kp = kt[p];
            double *Sp = S + (size_t)p * D;
            for (int c = 0; c < D; ++c) Sp[c] += kp * vt[c];
            z[p] += kp;
        }
        double den = 0.0;
        for (int p = 0; p < D; ++p) den += qt[p] * z[p];
        if (!(den > 0.0)) bad = 1;
        double *ot = o + (size_t)t * D;
        for (int c = 0; c < D; ++c) ot[c] = 0.0;
        for (int p = 0; p < D; ++p) {
            double qp = qt[p];
            const double *Sp = S + (size_t)p * D;
            for (int c = 0; c < D; ++c) ot[c] += qp * Sp[c];
        }
        for (int c = 0; c < D; ++c) ot[c] /= den;
    }
    return bad;
}

int la_oracle_fwd(int G, int T, int D,
                  const double *q, const double *k, const double *v,
                  const double *S_in, const double *z_in,
                  double *o, double *S_out, double *z_out, int nthreads)
{
    if (G < 0 || T < 0 || D < 1 || !q || !k || !v || !o || !S_out || !z_out) return 1;
    if ((S_in == NULL) != (z_in == NULL)) return 1;
    set_threads(nthreads);
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int g = 0; g < G; ++g) {
        size_t tok = (size_t)g * T * D, st = (size_t)g * D * D, zs = (size_t)g * D;
        double *S = S_out + st, *z = z_out + zs;
        if (S_in) {
            memcpy(S, S_in + st, sizeof(double) * (size_t)D * D);
            memcpy(z, z_in + zs, sizeof(double) * (size_t)D);
        } else {
            memset(S, 0, sizeof(double) * (size_t)D * D);
            memset(z, 0, sizeof(double) * (size_t)D);
        }
        bad |= fwd_group(T, D, q + tok, k + tok, v + tok, S, z, o + tok);
    }
    return bad ? 2 : 0;
}

/* One group's backward.  Scratch: S (D*D), z (D), dn (T*D), dden (T). */
static int bwd_group(int T, int D, const double *q, const double *k, const double *v,
                     const double *S_in, const double *z_in, const double *dO,
                     const double *dS_out, const double *dz_out,
                     double *dq, double *dk, double *dv, double *dS_in, double *dz_in,
                     double *S, double *z, double *dn, double *dden)
{
    int bad = 0;
    if (S_in) {
        memcpy(S, S_in, sizeof(double) * (size_t)D * D);
        memcpy(z, z_in, sizeof(double) * (size_t)D);
    } else {
        memset(S, 0, sizeof(double) * (size_t)D * D);
        memset(z, 0, sizeof(double) * (size_t)D);
    }
    /* forward sweep: rebuild S_t, z_t, o_t; form dn_t, dden_t and dq_t */
    for (int t = 0; t < T; ++t) {
        const double *qt = q + (size_t)t * D, *kt = k + (size_t)t * D, *vt = v + (size_t)t * D;
        const double *gt = dO + (size_t)t * D;
        for (int p = 0; p < D; ++p) {
            double kp = kt[p];
            double *Sp = S + (size_t)p * D;
            for (int c = 0; c < D; ++c) Sp[c] += kp * vt[c];
            z[p] += kp;
        }
        double den = 0.0;
        for (int p = 0; p < D; ++p) den += qt[p] * z[p];
        if (!(den > 0.0)) bad = 1;
        /* o_t and dO_t . o_t */
        double go = 0.0;
        for (int c = 0; c < D; ++c) {
            double n = 0.0;
            for (int p = 0; p < D; ++p) n += qt[p] * S[(size_t)p * D + c];
            go += gt[c] * (n / den);
        }
        double *dnt = dn + (size_t)t * D;
        for (int c = 0; c < D; ++c) dnt[c] = gt[c] / den;
        dden[t] = -go / den;
        double *dqt = dq + (size_t)t * D;
        for (int p = 0; p < D; ++p) {
            const double *Sp = S + (size_t)p * D;
            double acc = 0.0;
            for (int c = 0; c < D; ++c) acc += Sp[c] * dnt[c];
            dqt[p] = acc + dden[t] * z[p];
        }
    }
    /* reverse sweep: Sh, zh start from the upstream carry gradient */
    double *Sh = dS_in, *zh = dz_in;
    if (dS_out) {
        memcpy(Sh, dS_out, sizeof(double) * (size_t)D * D);
        memcpy(zh, dz_out, sizeof(double) * (size_t)D);
    } else {
        memset(Sh, 0, sizeof(double) * (size_t)D * D);
        memset(zh, 0, sizeof(double) * (size_t)D);
    }
    for (int t = T - 1; t >= 0; --t) {
        const double *qt = q + (size_t)t * D, *kt = k + (size_t)t * D, *vt = v + (size_t)t * D;
        const double *dnt = dn + (size_t)t * D;
        for (int p = 0; p < D; ++p) {
            double qp = qt[p];
            double *Shp = Sh + (size_t)p * D;
            for (int c = 0; c < D; ++c) Shp[c] += qp * dnt[c];
            zh[p] += dden[t] * qp;
        }
        double *dkt = dk + (size_t)t * D, *dvt = dv + (size_t)t * D;
        for (int p = 0; p < D; ++p) {
            const double *Shp = Sh + (size_t)p * D;
            double acc = 0.0;
            for (int c = 0; c < D; ++c) acc += Shp[c] * vt[c];
            dkt[p] = acc + zh[p];
        }
        for (int c = 0; c < D; ++c) dvt[c] = 0.0;
        for (int p = 0; p < D; ++p) {
            double kp = kt[p];
            const double *Shp = Sh + (size_t)p * D;
            for (int c = 0; c < D; ++c) dvt[c] += Shp[c] * kp;
        }
    }
    return bad;
}

int la_oracle_bwd(int G, int T, int D,
                  const double *q, const double *k, const double *v,
                  const double *S_in, const double *z_in, const double *dO,
                  const double *dS_out, const double *dz_out,
                  double *dq, double *dk, double *dv, double *dS_in, double *dz_in, int nthreads)
{
    if (G < 0 || T < 0 || D < 1 || !q || !k || !v || !dO || !dq || !dk || !dv || !dS_in || !dz_in)
        return 1;
    if ((S_in == NULL) != (z_in == NULL)) return 1;
    if ((dS_out == NULL) != (dz_out == NULL)) return 1;
    set_threads(nthreads);
    int bad = 0, oom = 0;
#pragma omp parallel reduction(| : bad, oom)
    {
        size_t scratch = (size_t)D * D + D + (size_t)T * D + (size_t)T;
        double *buf = (double *)malloc(sizeof(double) * (scratch ? scratch : 1));
        if (!buf) {
            oom = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int g = 0; g < G; ++g) {
            if (!buf) continue;
            size_t tok = (size_t)g * T * D, st = (size_t)g * D * D, zs = (size_t)g * D;
            double *S = buf, *z = S + (size_t)D * D, *dn = z + D, *dden = dn + (size_t)T * D;
            bad |= bwd_group(T, D, q + tok, k + tok, v + tok,
                             S_in ? S_in + st : NULL, z_in ? z_in + zs : NULL, dO + tok,
                             dS_out ? dS_out + st : NULL, dz_out ? dz_out + zs : NULL,
                             dq + tok, dk + tok, dv + tok, dS_in + st, dz_in + zs,
                             S, z, dn, dden);
        }
        free(buf);
    }
    if (oom) return 1;
    return bad ? 2 : 0;
}
