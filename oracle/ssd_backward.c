/*
 * CPU oracle for the gradient of the SSD layer: reverse-mode differentiation
 * of the plain sequential recurrence, in float64.  TEST INFRASTRUCTURE ONLY:
 * nothing in the product path may link or call this file.
 *
 * Forward map (the same as ssd_recurrence.c; Mamba-2 review, docsaid.org,
 * section "SSM を一つの行列として書く"; SSD summary page, section "SSD層"):
 *   a_t = exp(dt_t A_h),  h_t = a_t h_{t-1} + x_t B_t^T,  y_t = h_t C_t + D_h x_t,
 *   h_{-1} = init, final = h_{L-1}.
 * Given the output gradients dy [b, L, H, P] and dfinal [b, H, P, N] (NULL:
 * zero), the adjoint g_t = dLoss/dh_t runs backwards in time:
 *   g_{L-1} = dfinal;  for t = L-1 .. 0:
 *     g_t      += dy_t C_t^T                       (y_t reads h_t)
 *     dC_t     += h_t^T dy_t                        (per head; summed over the group)
 *     dx_t      = g_t B_t + D_h dy_t
 *     dB_t     += g_t^T x_t                         (per head; summed over the group)
 *     da_t      = <g_t, h_{t-1}>                     (Frobenius product)
 *     ddt_t     = da_t a_t A_h,   dA_h += da_t a_t dt_t,   dD_h += dy_t . x_t
 *     g_{t-1}   = a_t g_t
 *   dinit = g_{-1}.
 * Each step is the chain rule applied to one line of the forward map, in
 * reverse order; nothing is blocked or reordered.
 *
 * States are kept every K = 64 steps on the way forward and recomputed
 * inside each segment on the way back, so memory is O(K P N) per sequence.
 *
 * Outputs (row-major): dx [b, L, H, P], ddt [b, L, H], dB_h and dC_h
 * [b, L, H, N] (the contribution of each head; the caller sums the heads of
 * each group), dA_bh and dD_bh [b, H] (per batch; the caller sums over b),
 * dinit [b, H, P, N] (may be NULL).  Every (b, h) sequence is independent;
 * OpenMP runs them in parallel.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define SEG 64

static int run_backward(int64_t b, int64_t h, int64_t L, int64_t H, int64_t P, int64_t N, int64_t G,
                        const double *x, const double *dt, const double *A, const double *B,
                        const double *C, const double *D, const double *init, const double *dy,
                        const double *dfinal, double *dx, double *ddt, double *dB_h, double *dC_h,
                        double *dA_bh, double *dD_bh, double *dinit) {
    const int64_t g = h / (H / G);
    const double Ah = A[h];
    const double Dh = D ? D[h] : 0.0;
    const int64_t PN = P * N;
    const int64_t nseg = (L + SEG - 1) / SEG;
    /* ck[s] = state entering segment s (h_{s SEG - 1}); seg[k] = h_{s SEG + k}; gst = adjoint */
    double *ck = (double *)malloc(sizeof(double) * (size_t)(nseg > 0 ? nseg : 1) * PN);
    double *seg = (double *)malloc(sizeof(double) * SEG * PN);
    double *state = (double *)malloc(sizeof(double) * PN);
    double *gst = (double *)malloc(sizeof(double) * PN);
    if (!ck || !seg || !state || !gst) {
        free(ck); free(seg); free(state); free(gst);
        return 1;
    }
    /* forward pass: checkpoints only */
    for (int64_t i = 0; i < PN; ++i) state[i] = init ? init[(b * H + h) * PN + i] : 0.0;
    for (int64_t t = 0; t < L; ++t) {
        if (t % SEG == 0) memcpy(ck + (t / SEG) * PN, state, sizeof(double) * PN);
        const double a = exp(dt[(b * L + t) * H + h] * Ah);
        const double *xt = x + ((b * L + t) * H + h) * P;
        const double *Bt = B + ((b * L + t) * G + g) * N;
        for (int64_t p = 0; p < P; ++p)
            for (int64_t n = 0; n < N; ++n) state[p * N + n] = a * state[p * N + n] + xt[p] * Bt[n];
    }
    for (int64_t i = 0; i < PN; ++i) gst[i] = dfinal ? dfinal[(b * H + h) * PN + i] : 0.0;
    double dA = 0.0, dD = 0.0;
    /* backward pass, segment by segment */
    for (int64_t s = nseg - 1; s >= 0; --s) {
        const int64_t t0 = s * SEG, t1 = (t0 + SEG < L) ? t0 + SEG : L;
        /* recompute h_t for t in [t0, t1) */
        memcpy(state, ck + s * PN, sizeof(double) * PN);
        for (int64_t t = t0; t < t1; ++t) {
            const double a = exp(dt[(b * L + t) * H + h] * Ah);
            const double *xt = x + ((b * L + t) * H + h) * P;
            const double *Bt = B + ((b * L + t) * G + g) * N;
            double *ht = seg + (t - t0) * PN;
            for (int64_t p = 0; p < P; ++p)
                for (int64_t n = 0; n < N; ++n) {
                    state[p * N + n] = a * state[p * N + n] + xt[p] * Bt[n];
                    ht[p * N + n] = state[p * N + n];
                }
        }
        for (int64_t t = t1 - 1; t >= t0; --t) {
            const double dtt = dt[(b * L + t) * H + h];
            const double a = exp(dtt * Ah);
            const double *xt = x + ((b * L + t) * H + h) * P;
            const double *Bt = B + ((b * L + t) * G + g) * N;
            const double *Ct = C + ((b * L + t) * G + g) * N;
            const double *dyt = dy + ((b * L + t) * H + h) * P;
            const double *ht = seg + (t - t0) * PN;
            const double *hprev = (t > t0) ? seg + (t - t0 - 1) * PN : ck + s * PN;
            double *dxt = dx + ((b * L + t) * H + h) * P;
            double *dBt = dB_h + ((b * L + t) * H + h) * N;
            double *dCt = dC_h + ((b * L + t) * H + h) * N;
            /* g_t += dy_t C_t^T */
            for (int64_t p = 0; p < P; ++p)
                for (int64_t n = 0; n < N; ++n) gst[p * N + n] += dyt[p] * Ct[n];
            /* dC_t = h_t^T dy_t */
            for (int64_t n = 0; n < N; ++n) {
                double acc = 0.0;
                for (int64_t p = 0; p < P; ++p) acc += ht[p * N + n] * dyt[p];
                dCt[n] = acc;
            }
            /* dx_t = g_t B_t + D dy_t;  dD += dy_t . x_t */
            for (int64_t p = 0; p < P; ++p) {
                double acc = 0.0;
                for (int64_t n = 0; n < N; ++n) acc += gst[p * N + n] * Bt[n];
                dxt[p] = acc + Dh * dyt[p];
                dD += dyt[p] * xt[p];
            }
            /* dB_t = g_t^T x_t */
            for (int64_t n = 0; n < N; ++n) {
                double acc = 0.0;
                for (int64_t p = 0; p < P; ++p) acc += gst[p * N + n] * xt[p];
                dBt[n] = acc;
            }
            /* da_t = <g_t, h_{t-1}>;  a_t = exp(dt A): d a / d dt = a A, d a / d A = a dt */
            double da = 0.0;
            for (int64_t i = 0; i < PN; ++i) da += gst[i] * hprev[i];
            ddt[(b * L + t) * H + h] = da * a * Ah;
            dA += da * a * dtt;
            /* g_{t-1} = a_t g_t */
            for (int64_t i = 0; i < PN; ++i) gst[i] *= a;
        }
    }
    if (dinit) memcpy(dinit + (b * H + h) * PN, gst, sizeof(double) * PN);
    dA_bh[b * H + h] = dA;
    dD_bh[b * H + h] = dD;
    free(ck); free(seg); free(state); free(gst);
    return 0;
}

int ssd_oracle_backward(int64_t batch, int64_t L, int64_t H, int64_t P, int64_t N, int64_t G,
                        const double *x, const double *dt, const double *A, const double *B,
                        const double *C, const double *D, const double *init, const double *dy,
                        const double *dfinal, double *dx, double *ddt, double *dB_h, double *dC_h,
                        double *dA_bh, double *dD_bh, double *dinit) {
    if (batch < 0 || L < 0 || H <= 0 || P <= 0 || N <= 0 || G <= 0 || H % G) return 1;
    int err = 0;
#pragma omp parallel for schedule(dynamic) reduction(| : err)
    for (int64_t bh = 0; bh < batch * H; ++bh)
        err |= run_backward(bh / H, bh % H, L, H, P, N, G, x, dt, A, B, C, D, init, dy, dfinal, dx, ddt,
                            dB_h, dC_h, dA_bh, dD_bh, dinit);
    return err;
}
