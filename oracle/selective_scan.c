/*
 * CPU oracle for the selective scan (the Mamba-1 scan), float64.  TEST
 * INFRASTRUCTURE ONLY: nothing in the product path may link or call this file.
 *
 * Mamba review page (youngju.dev), section 3.3: per channel d with a diagonal
 * state matrix A[d, :] (N entries), step size delta_t, and inputs B_t, C_t,
 *   h_t[n] = exp(delta_t A[d, n]) h_{t-1}[n] + delta_t B_t[n] x_t[d]
 *   y_t[d] = sum_n C_t[n] h_t[n]
 * and the block of section 3.4 around it: the skip term D[d] x_t[d] and the
 * output multiplied by SiLU of the gate branch z.  Section 3.1: the step size
 * is a softplus of a linear map, whose bias is delta_bias.  So per (b, d):
 *   dl  = delta + delta_bias[d];  dl = softplus(dl) if softplus
 *   h   = exp(dl A[d, :]) * h + dl x B_t       (h_{-1} = init or 0)
 *   out = (C_t . h + D[d] x) * silu(z)          (no gate when z is NULL)
 * B, C are [b, L, G, N], channel d reads group d / (Dch / G).  Layouts:
 * x, delta, z, y [b, L, Dch]; A [Dch, N]; D, delta_bias [Dch]; states
 * [b, Dch, N].  D, z, delta_bias, init, final nullable.  OpenMP over (b, d).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

static double softplus(double v) { return v > 30.0 ? v + log1p(exp(-v)) : log1p(exp(v)); }

int ssd_oracle_selective_scan(int64_t batch, int64_t L, int64_t Dch, int64_t N, int64_t G,
                              const double *x, const double *delta, const double *A,
                              const double *B, const double *C, const double *D, const double *z,
                              const double *delta_bias, int64_t use_softplus, const double *init,
                              double *y, double *final_state) {
    if (batch < 0 || L < 0 || Dch <= 0 || N <= 0 || G <= 0 || Dch % G) return 1;
    int err = 0;
#pragma omp parallel for schedule(static) reduction(| : err)
    for (int64_t bd = 0; bd < batch * Dch; ++bd) {
        const int64_t b = bd / Dch, d = bd % Dch, g = d / (Dch / G);
        double *h = (double *)malloc(sizeof(double) * N);
        if (!h) {
            err |= 1;
            continue;
        }
        for (int64_t n = 0; n < N; ++n) h[n] = init ? init[(b * Dch + d) * N + n] : 0.0;
        for (int64_t t = 0; t < L; ++t) {
            const int64_t i = (b * L + t) * Dch + d;
            double dl = delta[i] + (delta_bias ? delta_bias[d] : 0.0);
            if (use_softplus) dl = softplus(dl);
            const double xv = x[i];
            const double *Bt = B + ((b * L + t) * G + g) * N;
            const double *Ct = C + ((b * L + t) * G + g) * N;
            double acc = 0.0;
            for (int64_t n = 0; n < N; ++n) {
                h[n] = exp(dl * A[d * N + n]) * h[n] + dl * Bt[n] * xv;
                acc += Ct[n] * h[n];
            }
            double out = acc + (D ? D[d] : 0.0) * xv;
            if (z) out *= z[i] / (1.0 + exp(-z[i]));
            y[i] = out;
        }
        if (final_state)
            for (int64_t n = 0; n < N; ++n) final_state[(b * Dch + d) * N + n] = h[n];
        free(h);
    }
    return err;
}
