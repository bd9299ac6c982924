/*
 * CPU oracle for the SSD (state space dual) layer: the plain sequential
 * recurrence in float64.  TEST INFRASTRUCTURE ONLY: nothing in the product
 * path may link or call this file; it exists so the tests, the smoke check
 * and the CPU-baseline leg of the benchmark have an independent answer.
 *
 * What it computes (Mamba-2 review, docsaid.org "Mamba-2", section
 * "SSM を一つの行列として書く", first display: h_t = A_t h_{t-1} + B_t x_t,
 * y_t = C_t^T h_t; section "A を一つの数に簡略化する": A_t = a_t I with a
 * scalar a_t in [0, 1] per step; the SSD summary page, section "SSD層", the
 * scalar recurrence h_t = a_t h_{t-1} + B_t x_t), written per head with a
 * state matrix of P rows (one per input channel of the head) and N columns:
 *
 *   a_t      = exp(dt[b,t,h] * A[h])
 *   h_{-1}   = init[b,h]            (zeros when init == NULL)
 *   h_t[p,n] = a_t * h_{t-1}[p,n] + x[b,t,h,p] * B[b,t,g,n]
 *   y[b,t,h,p] = sum_n h_t[p,n] * C[b,t,g,n] + D[h] * x[b,t,h,p]
 *   final[b,h] = h_{L-1}
 *
 * with group g = h / (H / G).  The decay a_t = exp(dt * A) is the
 * zero-order-hold decay of the discretisation (Mamba review page, section
 * 2.2; state-space guide page, equation (2)); the input is added without a
 * dt factor, as in the SSD form above.  D is the per-head skip term.
 *
 * Optionally it also reports the state entering every chunk of Q steps:
 * bnd[b, c, h] = h_{cQ-1} (bnd[b, 0, h] = init), which is what the
 * inter-chunk state passing of the chunked algorithm must hand to chunk c.
 *
 * Layouts (row-major, contiguous):
 *   x, y [b, L, H, P]; dt [b, L, H]; B, C [b, L, G, N]; A, D [H];
 *   init, final [b, H, P, N]; bnd [b, nc, H, P, N] with nc = ceil(L / Q).
 *
 * Every (b, h) sequence is independent; OpenMP runs them in parallel.  No
 * blocking, reordering or fast-math: each step is done in the order above.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

int ssd_oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void ssd_oracle_set_num_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* One (b, h) sequence over t in [0, L). h is the P x N state, updated in place. */
static void run_sequence(int64_t b, int64_t h, int64_t L, int64_t H, int64_t P, int64_t N,
                         int64_t G, const double *x, const double *dt, const double *A,
                         const double *B, const double *C, const double *D, double *state,
                         double *y, int64_t Q, double *bnd) {
    const int64_t g = h / (H / G);
    const double Ah = A[h];
    const double Dh = D ? D[h] : 0.0;
    const int64_t nc = Q > 0 ? (L + Q - 1) / Q : 0;
    for (int64_t t = 0; t < L; ++t) {
        if (bnd && t % Q == 0) {
            const int64_t c = t / Q;
            memcpy(bnd + ((b * nc + c) * H + h) * P * N, state, sizeof(double) * P * N);
        }
        const double a = exp(dt[(b * L + t) * H + h] * Ah);
        const double *xt = x + ((b * L + t) * H + h) * P;
        const double *Bt = B + ((b * L + t) * G + g) * N;
        const double *Ct = C + ((b * L + t) * G + g) * N;
        double *yt = y + ((b * L + t) * H + h) * P;
        for (int64_t p = 0; p < P; ++p) {
            double *hp = state + p * N;
            double acc = 0.0;
            for (int64_t n = 0; n < N; ++n) {
                hp[n] = a * hp[n] + xt[p] * Bt[n];
                acc += hp[n] * Ct[n];
            }
            yt[p] = acc + Dh * xt[p];
        }
    }
}

/* Forward over a whole sequence.  Returns 0, or -1 on a bad shape. */
int ssd_oracle_forward(int64_t batch, int64_t L, int64_t H, int64_t P, int64_t N, int64_t G,
                       const double *x, const double *dt, const double *A, const double *B,
                       const double *C, const double *D, const double *init, double *y,
                       double *final_state, int64_t Q, double *bnd) {
    if (batch < 0 || L < 0 || H <= 0 || P <= 0 || N <= 0 || G <= 0 || H % G != 0) return -1;
    if (bnd && Q <= 0) return -1;
    const int64_t BH = batch * H;
#pragma omp parallel
    {
        double *state = (double *)malloc(sizeof(double) * P * N);
#pragma omp for schedule(dynamic, 1)
        for (int64_t bh = 0; bh < BH; ++bh) {
            const int64_t b = bh / H, h = bh % H;
            if (init)
                memcpy(state, init + bh * P * N, sizeof(double) * P * N);
            else
                memset(state, 0, sizeof(double) * P * N);
            run_sequence(b, h, L, H, P, N, G, x, dt, A, B, C, D, state, y, Q, bnd);
            if (final_state) memcpy(final_state + bh * P * N, state, sizeof(double) * P * N);
        }
        free(state);
    }
    return 0;
}

/*
 * One decode step: a single iteration of the recurrence above applied to a
 * carried state (Mamba-2 review page, section "4つのトークンで計算してみる":
 * the recurrent route keeps only the state and suits generation).
 * state [b, H, P, N] is updated in place; x, y [b, H, P]; dt [b, H];
 * B, C [b, G, N].
 */
int ssd_oracle_decode_step(int64_t batch, int64_t H, int64_t P, int64_t N, int64_t G,
                           double *state, const double *x, const double *dt, const double *A,
                           const double *B, const double *C, const double *D, double *y) {
    if (batch < 0 || H <= 0 || P <= 0 || N <= 0 || G <= 0 || H % G != 0) return -1;
    const int64_t BH = batch * H;
#pragma omp parallel for schedule(static)
    for (int64_t bh = 0; bh < BH; ++bh) {
        const int64_t b = bh / H, h = bh % H;
        /* A decode step is the recurrence with L = 1 on this (b, h). */
        run_sequence(0, 0, 1, 1, P, N, 1, x + bh * P, dt + bh, A + h, B + (b * G + h / (H / G)) * N,
                     C + (b * G + h / (H / G)) * N, D ? D + h : NULL, state + bh * P * N,
                     y + bh * P, 0, NULL);
    }
    return 0;
}
