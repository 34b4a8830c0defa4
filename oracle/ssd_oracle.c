/*
 * ssd_oracle.c -- fp64 CPU oracle for the Mamba-2 SSD (structured state space
 * duality) scan.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file; only the tests, the smoke check and the benchmark's CPU
 * baseline use it.  It shares no code, header or constant with the HIP path.
 *
 * What it computes (the plain definition, token by token, in double):
 *
 *   per (batch b, head h), with group g = h / (H / G):
 *     S <- init[b, h]            (P x N; zeros when no initial state is given)
 *     for t = 0 .. L-1:
 *       alpha = exp(dt[b,t,h] * A[h])
 *       S[p,n] <- alpha * S[p,n] + dt[b,t,h] * x[b,t,h,p] * Bm[b,t,g,n]
 *       y[b,t,h,p] = sum_n S[p,n] * Cm[b,t,g,n] + D[h] * x[b,t,h,p]
 *     final[b, h] = S
 *
 * This is the selective SSM recurrence h_t = A_t h_{t-1} + B_t x_t,
 * y_t = C_t^T h_t of the "Mamba-2" note (section "writing the SSM as a
 * matrix"), specialised to a scalar decay a_t = exp(dt_t * A_h) times the
 * identity (section "reducing A to a number", the SSD case), with the input
 * term discretised as dt_t * B_t (the decay is the zero-order-hold
 * exp(dt A) of the "Mamba" reading notes, section 2.2), with several heads of
 * dimension P sharing B and C within a group (section "Mamba-2 block", item 2),
 * and with a skip term D_h * x_t.
 *
 * Layouts (dense, row-major): x, y [B,L,H,P]; dt [B,L,H]; A, D [H];
 * Bm, Cm [B,L,G,N]; init, final [B,H,P,N].  For the step form, x and y are
 * [B,H,P], dt is [B,H] and Bm, Cm are [B,G,N].
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Token-by-token recurrence over whole sequences.  When bh_list is non-NULL,
 * only the listed (b * H + h) pairs are computed; y and final_state of the
 * other pairs are left untouched.  Returns 0, or -1 on bad arguments or when
 * out of memory. */
int oracle_ssd_recurrence(int64_t Bsz, int64_t L, int64_t H, int64_t P, int64_t G, int64_t N,
                          const double *x, const double *dt, const double *A,
                          const double *Bm, const double *Cm, const double *D,
                          const double *init, double *y, double *final_state,
                          const int64_t *bh_list, int64_t n_bh)
{
    if (Bsz < 0 || L < 0 || H <= 0 || P <= 0 || G <= 0 || N <= 0 || H % G != 0)
        return -1;
    const int64_t npairs = bh_list ? n_bh : Bsz * H;
    const int64_t heads_per_group = H / G;
    int failed = 0;

#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t k = 0; k < npairs; ++k) {
        const int64_t bh = bh_list ? bh_list[k] : k;
        if (bh < 0 || bh >= Bsz * H) { failed = 1; continue; }
        const int64_t b = bh / H, h = bh % H, g = h / heads_per_group;
        double *S = (double *)malloc((size_t)(P * N) * sizeof(double));
        if (!S) { failed = 1; continue; }
        if (init)
            memcpy(S, init + bh * P * N, (size_t)(P * N) * sizeof(double));
        else
            memset(S, 0, (size_t)(P * N) * sizeof(double));

        for (int64_t t = 0; t < L; ++t) {
            const double dtv = dt[(b * L + t) * H + h];
            const double alpha = exp(dtv * A[h]);
            const double *xt = x + ((b * L + t) * H + h) * P;
            const double *bt = Bm + ((b * L + t) * G + g) * N;
            const double *ct = Cm + ((b * L + t) * G + g) * N;
            double *yt = y + ((b * L + t) * H + h) * P;
            for (int64_t p = 0; p < P; ++p) {
                double *row = S + p * N;
                const double u = dtv * xt[p];
                double acc = 0.0;
                for (int64_t n = 0; n < N; ++n) {
                    row[n] = alpha * row[n] + u * bt[n];
                    acc += row[n] * ct[n];
                }
                yt[p] = acc + D[h] * xt[p];
            }
        }
        if (final_state)
            memcpy(final_state + bh * P * N, S, (size_t)(P * N) * sizeof(double));
        free(S);
    }
    return failed ? -1 : 0;
}

/* One decode token: the same update applied once, in place on state
 * [B,H,P,N], with the output read from the updated state.  bh_list as above. */
int oracle_ssd_step(int64_t Bsz, int64_t H, int64_t P, int64_t G, int64_t N,
                    double *state, const double *x, const double *dt, const double *A,
                    const double *Bm, const double *Cm, const double *D, double *y,
                    const int64_t *bh_list, int64_t n_bh)
{
    if (Bsz < 0 || H <= 0 || P <= 0 || G <= 0 || N <= 0 || H % G != 0)
        return -1;
    const int64_t npairs = bh_list ? n_bh : Bsz * H;
    const int64_t heads_per_group = H / G;
    int failed = 0;

#pragma omp parallel for schedule(static)
    for (int64_t k = 0; k < npairs; ++k) {
        const int64_t bh = bh_list ? bh_list[k] : k;
        if (bh < 0 || bh >= Bsz * H) { failed = 1; continue; }
        const int64_t b = bh / H, h = bh % H, g = h / heads_per_group;
        const double dtv = dt[b * H + h];
        const double alpha = exp(dtv * A[h]);
        const double *xv = x + (b * H + h) * P;
        const double *bv = Bm + (b * G + g) * N;
        const double *cv = Cm + (b * G + g) * N;
        double *S = state + bh * P * N;
        for (int64_t p = 0; p < P; ++p) {
            double *row = S + p * N;
            const double u = dtv * xv[p];
            double acc = 0.0;
            for (int64_t n = 0; n < N; ++n) {
                row[n] = alpha * row[n] + u * bv[n];
                acc += row[n] * cv[n];
            }
            y[(b * H + h) * P + p] = acc + D[h] * xv[p];
        }
    }
    return failed ? -1 : 0;
}
