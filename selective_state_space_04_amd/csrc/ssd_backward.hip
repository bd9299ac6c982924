// Gradient of the SSD layer (gfx950 / MI355X), by the chunked algorithm.
//
// Forward map per batch row b, head h (group g), chunk c of q steps starting
// at s, with cs_i the decay prefix inside the chunk and H_c the state entering
// it (Mamba-2 review, docsaid.org, sections "A を一つの数に簡略化する" and
// "2つのルートを半分ずつ"):
//   y_i      = sum_{j<=i} M_ij x_j + exp(cs_i) H_c C_i + D x_i,   M_ij = exp(cs_i - cs_j) C_i.B_j
//   H_{c+1}  = exp(cs_e) H_c + sum_j exp(cs_e - cs_j) x_j B_j^T     (e = q - 1)
// Given dy and dfinal = dLoss/dH_nc, the chain rule gives, with
// R_c = dLoss/dH_{c+1} (the gradient of the state leaving chunk c):
//   R_{nc-1} = dfinal,  R_{c-1} = exp(cs_e(c)) R_c + sum_i exp(cs_i) dy_i C_i^T,  dinit = R_{-1}
//   dx_j = sum_{i>=j} M_ij dy_i + exp(cs_e - cs_j) R_c B_j + D dy_j
//   dC_i = sum_h [ sum_{j<=i} exp(cs_i - cs_j)(dy_i.x_j) B_j + exp(cs_i) H_c^T dy_i ]
//   dB_j = sum_h [ sum_{i>=j} exp(cs_i - cs_j)(dy_i.x_j) C_i + exp(cs_e - cs_j) R_c^T x_j ]
// and for the log-decays, with y'_k = y_k - D x_k and dx'_k = dx_k - D dy_k,
//   dLoss/dcs_k = dy_k.y'_k - x_k.dx'_k + [k = e] <R_c, H_{c+1}>
// (differentiate each exponent: the terms in which cs_k appears with a plus
// sign sum to dy_k.y'_k plus the end-of-chunk state, those with a minus sign
// to x_k.dx'_k), so the gradient of dA_t = dt_t A_h, which enters every cs_k
// with k >= t, is the suffix sum ddA_t = sum_{k>=t} dLoss/dcs_k, and
// ddt_t = A_h ddA_t, dA_h = sum dt_t ddA_t, dD_h = sum dy.x.
//
// Two choices keep the decay gradients accurate where a head forgets fast
// (|cs| in the thousands, neighbouring decays ~1e-3): the diagonal terms
// M_kk x_k and M_kk dy_k, which cancel exactly between dy_k.y'_k and
// x_k.dx'_k, are left out of both (strict masks; M_kk dy_k is added to dx on
// its own); and for float32 inputs the prefix is kept in float64 (dt A is
// exact there), so cs_i - cs_j is exact before it is rounded for exp.
//
// Kernels (the forward states H_c and the state gradients R_c are produced
// first by the step kernels of ssd_kernels.hip and k_state_passing_rev):
//   k_bwd_frags     per (b, c, g, 16-row tile), bf16: C B^T, C and B in the
//                   fragment order k_chunk_bwd_pf loads (else k_chunk_cb of
//                   ssd_kernels.hip writes C B^T and its transpose row-major).
//   k_chunk_bwd     per (b, c, h): recomputes y'_i, computes dx and the
//                   decay gradients of the chunk; per-chunk partial sums of
//                   dA_h and dD_h (k_chunk_bwd_pf: the bf16 version with each
//                   tile's operands loaded one tile ahead).
//   k_group_bwd     per (b, c, g, 64 rows): loops over the heads of the group
//                   and sums exp(cs_i - cs_j)(dy_i.x_j) (dCB, both
//                   orientations) and the state terms of dC and dB (float32
//                   inputs, and bf16 shapes with N = 256 or P N > 8192).
//   k_group_dcb_rb, the same sums for the other bf16 shapes, split so each
//   k_group_dcb,    kernel's accumulators stay in registers at several waves
//   k_group_state   per SIMD: dCB per 64-row block (k_group_dcb_rb, P 32 or
//                   64) or per 64 x 64 block pair (k_group_dcb), the state
//                   terms per 128 rows with each head's state in LDS.
//   k_group_combine per (b, c, g, 64 rows): dC = dC_state + dCB B,
//                   dB = dB_state + dCB^T C, rounded to the input dtype.
//   k_head_reduce   per h: sums the per-chunk partials of dA_h and dD_h.
#include <type_traits>

#include "ssd_device.h"
#include "ssd_launch.h"

namespace ssd {

// ---------------------------------------------------------------------------
// Reverse inter-chunk recurrence, in place: on entry S[c] = sum_i exp(cs_i)
// dy_i C_i^T of chunk c; on return S[c] = R_c.  Mirror image of
// k_state_passing: each thread owns four state elements of one (b, h) and
// walks the chunks from the last to the first, 8 chunk inputs loaded ahead.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_state_passing_rev(float *__restrict__ S,
                                                           const float *__restrict__ cs,
                                                           const float *dfinal, float *dinit,
                                                           int64_t L, int H, int PN, int Q,
                                                           int nc) {
    const int h = blockIdx.y;
    const int64_t b = blockIdx.z;
    const int e0 = (blockIdx.x * 256 + threadIdx.x) * 4;
    if (e0 >= PN) return;
    const int64_t bh = b * H + h;
    f32x4 gv = dfinal ? *(const f32x4 *)(dfinal + bh * PN + e0) : f32x4{0.f, 0.f, 0.f, 0.f};
    const float *csb = cs + bh * (int64_t)nc * Q;
    constexpr int U = 8;
    for (int c1 = nc - 1; c1 >= 0; c1 -= U) {
        f32x4 sv[U];
        float lam[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = c1 - u;
            if (c >= 0) {
                const int last = (int)min<int64_t>(Q, L - (int64_t)c * Q) - 1;
                lam[u] = __expf(csb[(int64_t)c * Q + last]);
                sv[u] = *(const f32x4 *)(S + (((b * nc + c) * H + h) * (int64_t)PN) + e0);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = c1 - u;
            if (c >= 0) {
                *(f32x4 *)(S + (((b * nc + c) * H + h) * (int64_t)PN) + e0) = gv;
                gv = lam[u] * gv + sv[u];
            }
        }
    }
    if (dinit) *(f32x4 *)(dinit + bh * PN + e0) = gv;
}

// ---------------------------------------------------------------------------
// Decay prefix in float64, one wave per (b, h, c): the same sums as
// k_chunk_cumsum, with dt A formed exactly (a float32 product fits in a
// float64 significand) and accumulated in float64.  Entries past a short
// chunk's end repeat its last value.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(64) void k_chunk_cumsum64(const T *__restrict__ dt,
                                                       const float *__restrict__ A,
                                                       double *__restrict__ cs, int64_t L, int H,
                                                       int Q, int nc) {
    const int c = blockIdx.x, h = blockIdx.y;
    const int64_t b = blockIdx.z;
    const int lane = threadIdx.x;
    const int64_t s = (int64_t)c * Q;
    const int q = (int)min<int64_t>(Q, L - s);
    const double Ah = A[h];
    const int per = (Q + 63) / 64;  // <= 4
    double v[4];
    double run = 0.0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int i = lane * per + e;
        double d = 0.0;
        if (e < per && i < q) d = (double)to_f32(dt[((b * L) + s + i) * H + h]) * Ah;
        run += d;
        v[e] = run;
    }
    double tot = run;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const double o = __shfl_up(tot, off, 64);
        if (lane >= off) tot += o;
    }
    const double excl = tot - run;
    double *out = cs + (((int64_t)b * H + h) * nc + c) * Q;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int i = lane * per + e;
        if (e < per && i < Q) out[i] = v[e] + excl;
    }
}

// exp(a - b) with the difference formed in the prefix's own precision.
template <typename CsT>
__device__ __forceinline__ float exp_diff(CsT a, CsT b) {
    return __expf((float)(a - b));
}

// fp32 [P][N] state -> bf16 [P][ld] in LDS.
template <int P, int N>
__device__ __forceinline__ void stage_state_bf16(const float *__restrict__ src, bf16 *dst, int ld) {
    for (int idx = threadIdx.x; idx < P * N / 8; idx += blockDim.x) {
        const int p = idx / (N / 8), n0 = (idx - p * (N / 8)) * 8;
        const f32x4 a0 = *(const f32x4 *)(src + (int64_t)p * N + n0);
        const f32x4 a1 = *(const f32x4 *)(src + (int64_t)p * N + n0 + 4);
        bf16x8 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            v[e] = (bf16)a0[e];
            v[e + 4] = (bf16)a1[e];
        }
        *(bf16x8 *)(dst + p * ld + n0) = v;
    }
}

// Four consecutive channels p0..p0+3 of one row, as float.
template <typename T>
__device__ __forceinline__ f32x4 load4(const T *p) {
    if constexpr (sizeof(T) == 2) {
        const u32x2 w = *(const u32x2 *)p;
        const bf16 *e = (const bf16 *)&w;
        return f32x4{(float)e[0], (float)e[1], (float)e[2], (float)e[3]};
    } else {
        return *(const f32x4 *)p;
    }
}

template <typename T>
__device__ __forceinline__ void store4(T *p, f32x4 v) {
    if constexpr (sizeof(T) == 2) {
        bf16 o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = (bf16)v[e];
        *(u32x2 *)p = *(const u32x2 *)o;
    } else {
        *(f32x4 *)p = v;
    }
}

__device__ __forceinline__ float dot4(f32x4 a, f32x4 b) {
    return a[0] * b[0] + a[1] * b[1] + a[2] * b[2] + a[3] * b[3];
}

// Sum over the four lane groups that share r = lane % 16.
__device__ __forceinline__ float sum_groups(float v) {
    v += __shfl_xor(v, 16, 64);
    v += __shfl_xor(v, 32, 64);
    return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// ---------------------------------------------------------------------------
// Per (b, c, h): dx, ddt and the chunk's partials of dA_h and dD_h.
// Two phases over the same LDS (bf16: one [P][Q] operand tile and one
// [P][N] state tile; f32: operands straight from global memory):
//   Y: x^T and H_c staged; per 16-row tile, Y''^T[p][i] = (H_c C_i) e^{cs_i}
//      + sum_{j<i} x^T[p][j] M_ij  (the forward's output without D and
//      without its diagonal term), then yy_i = dy_i . y''_i.
//   X: dy^T and R_c staged; per 16-column tile, dX''^T[p][j] =
//      e^{cs_e - cs_j} (R_c B_j) + sum_{i>j} dy^T[p][i] M_ij, with M read
//      from cbT so the step index i is contiguous; xdx_j = x_j . dx''_j and the
//      state part x_j . (e^{cs_e - cs_j} R_c B_j) summed for <R_c, H_{c+1}>;
//      dx = dx'' + (M_jj + D) dy stored.
// Then one wave forms dLoss/dcs_k, its suffix sums ddA, and writes ddt.
// Output tiles go to the waves in a snake order (triangular work balanced).
// ---------------------------------------------------------------------------
template <typename T, int P, int N, typename CsT>
__global__ __launch_bounds__(256) void k_chunk_bwd(
    const T *__restrict__ x, const T *__restrict__ dy, const T *__restrict__ dt,
    const float *__restrict__ A, const T *__restrict__ B, const T *__restrict__ C,
    const T *__restrict__ cb, const T *__restrict__ cbT, const CsT *__restrict__ cs,
    const float *__restrict__ Hs, const float *__restrict__ Rs, const float *__restrict__ D,
    T *__restrict__ dx, T *__restrict__ ddt, float *__restrict__ part, int64_t L, int H, int G,
    int Q, int nc) {
    constexpr bool BF = sizeof(T) == 2;
    constexpr int PT = P / 16;
    const int64_t wid = xcd_remap(blockIdx.x, gridDim.x);
    const int h = (int)(wid % H);
    const int64_t bc = wid / H;
    const int c = (int)(bc % nc);
    const int64_t b = bc / nc;
    const int g = h / (H / G);
    const int64_t s = (int64_t)c * Q;
    const int q = (int)min<int64_t>(Q, L - s);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int r = lane & 15, grp = lane >> 4;
    const int Qp = (Q + 31) & ~31;

    __shared__ CsT cs_s[256];
    __shared__ float yy_s[256], xdx_s[256], red_s[4][3];
    const CsT *csc = cs + (((int64_t)b * H + h) * nc + c) * Q;
    for (int j = threadIdx.x; j < 256; j += 256) {
        cs_s[j] = csc[min(j, Q - 1)];
        yy_s[j] = 0.f;
        xdx_s[j] = 0.f;
    }

    const int64_t row0 = (b * L + s) * H + h;  // (row of step s, head h) in x / dy / dx
    const T *Cb = C + ((b * L + s) * G + g) * N;
    const T *Bb = B + ((b * L + s) * G + g) * N;
    const int64_t cboff = (((int64_t)b * nc + c) * G + g) * (int64_t)Q * Q;
    const T *cbc = cb + cboff, *cbTc = cbT + cboff;
    const int64_t soff = (((int64_t)b * nc + c) * H + h) * (int64_t)P * N;
    const float *hp = Hs + soff, *rp = Rs + soff;
    const float Dh = D ? D[h] : 0.f;

    constexpr int XLD = 256 + 8, HLD = N + 8;
    __shared__ bf16 ops_s[BF ? P * XLD : 1];
    __shared__ bf16 st_s[BF ? P * HLD : 1];

    // State term of one 16-row (or column) tile: acc[pt][e] += sum_n S[p][n] V_row[n],
    // p = pt*16 + 4 grp + e, S = H_c or R_c, V_row the lane's row of C or B.
    auto state_term = [&](f32x4 *acc, const T *vrow, bool valid, const float *sg) {
        if constexpr (BF) {
#pragma unroll
            for (int k0 = 0; k0 < N; k0 += 32) {
                const int kk = k0 + grp * 8;
                const u32x4 z = {0u, 0u, 0u, 0u};
                const u32x4 bv = (valid && kk < N) ? *(const u32x4 *)(vrow + kk) : z;
#pragma unroll
                for (int pt = 0; pt < PT; ++pt) {
                    const u32x4 av = kk < N ? *(const u32x4 *)(st_s + (pt * 16 + r) * HLD + kk) : z;
                    acc[pt] = mfma_bf16(as_bf16x8(av), as_bf16x8(bv), acc[pt]);
                }
            }
        } else {
#pragma unroll 4
            for (int k0 = 0; k0 < N; k0 += 16) {
                const int kk = k0 + grp * 4;
                const f32x4 z = {0.f, 0.f, 0.f, 0.f};
                const f32x4 c4 = valid ? *(const f32x4 *)(vrow + kk) : z;
#pragma unroll
                for (int pt = 0; pt < PT; ++pt) {
                    const f32x4 h4 = *(const f32x4 *)(sg + (int64_t)(pt * 16 + r) * N + kk);
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[pt] = mfma_f32(h4[e], c4[e], acc[pt]);
                }
            }
        }
    };

    // ---------------- phase Y ----------------
    if constexpr (BF) {
        stage_transposed_bf16<false>((const bf16 *)x + row0 * P, (int64_t)H * P, Qp, P, q, ops_s,
                                     XLD, nullptr);
        stage_state_bf16<P, N>(hp, st_s, HLD);
    }
    __syncthreads();

    const int T16 = (q + 15) / 16;
    for (int round = 0; 4 * round < T16; ++round) {
        const int I = 4 * round + ((round & 1) ? 3 - wave : wave);
        if (I >= T16) continue;
        const int il = I * 16 + r;
        const bool vi = il < q;
        const CsT csi = cs_s[il];
        f32x4 acc[PT];
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) acc[pt] = f32x4{0.f, 0.f, 0.f, 0.f};
        state_term(acc, Cb + (int64_t)il * G * N, vi, hp);
        const float ei = __expf((float)csi);
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) acc[pt] *= ei;

        const T *grow = cbc + (int64_t)il * Q;
        const int jend = I * 16 + 15;
        if constexpr (BF) {
            for (int j0 = 0; j0 <= jend; j0 += 32) {
                const int jl = j0 + grp * 8;
                bf16x8 bm;
                if (jl < il) {
                    const bf16x8 gv = as_bf16x8(*(const u32x4 *)(grow + jl));
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int j = jl + e;
                        bm[e] = (bf16)((j < il) ? exp_diff(csi, cs_s[j]) * (float)gv[e] : 0.f);
                    }
                } else {
                    bm = as_bf16x8(u32x4{0u, 0u, 0u, 0u});
                }
#pragma unroll
                for (int pt = 0; pt < PT; ++pt) {
                    const bf16x8 ax = *(const bf16x8 *)(ops_s + (pt * 16 + r) * XLD + jl);
                    acc[pt] = mfma_bf16(ax, bm, acc[pt]);
                }
            }
        } else {
            for (int j0 = 0; j0 <= jend; j0 += 16) {
                const int jl = j0 + grp * 4;
                const f32x4 g4 = *(const f32x4 *)(grow + jl);
                float m[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int j = jl + e;
                    m[e] = (j < il) ? exp_diff(csi, cs_s[j]) * g4[e] : 0.f;
                }
#pragma unroll
                for (int pt = 0; pt < PT; ++pt) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int j = jl + e;
                        const float xa =
                            j < q ? to_f32(x[(row0 + (int64_t)j * H) * P + pt * 16 + r]) : 0.f;
                        acc[pt] = mfma_f32(xa, m[e], acc[pt]);
                    }
                }
            }
        }
        float yy = 0.f;
        if (vi) {
            const T *dyr = dy + (row0 + (int64_t)il * H) * P;
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) yy += dot4(acc[pt], load4(dyr + pt * 16 + 4 * grp));
        }
        yy = sum_groups(yy);
        if (grp == 0 && vi) yy_s[il] = yy;
    }
    __syncthreads();

    // ---------------- phase X ----------------
    if constexpr (BF) {
        stage_transposed_bf16<false>((const bf16 *)dy + row0 * P, (int64_t)H * P, Qp, P, q, ops_s,
                                     XLD, nullptr);
        stage_state_bf16<P, N>(rp, st_s, HLD);
    }
    float rh = 0.f;  // <R_c, H_c>
    for (int idx = threadIdx.x; idx < P * N / 4; idx += 256)
        rh += dot4(*(const f32x4 *)(rp + 4 * idx), *(const f32x4 *)(hp + 4 * idx));
    __syncthreads();

    const CsT csE = cs_s[q - 1];
    float vsum = 0.f, dDp = 0.f;
    for (int round = 0; 4 * round < T16; ++round) {
        const int J = 4 * round + ((round & 1) ? 3 - wave : wave);
        if (J >= T16) continue;
        const int jl = J * 16 + r;
        const bool vj = jl < q;
        const CsT csj = cs_s[jl];
        f32x4 acc[PT];
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) acc[pt] = f32x4{0.f, 0.f, 0.f, 0.f};
        state_term(acc, Bb + (int64_t)jl * G * N, vj, rp);
        const float wj = exp_diff(csE, csj);
        const T *xr = x + (row0 + (int64_t)jl * H) * P;
        f32x4 xv[PT];
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) {
            acc[pt] *= wj;
            xv[pt] = vj ? load4(xr + pt * 16 + 4 * grp) : f32x4{0.f, 0.f, 0.f, 0.f};
            vsum += dot4(acc[pt], xv[pt]);
        }

        const T *gcol = cbTc + (int64_t)jl * Q;  // cbT row j: M_ij / e^{cs_i - cs_j}, i contiguous
        if constexpr (BF) {
            for (int i0 = (J * 16) & ~31; i0 < q; i0 += 32) {
                const int il = i0 + grp * 8;
                bf16x8 bm;
                if (il + 7 > jl && il < q) {
                    const bf16x8 gv = as_bf16x8(*(const u32x4 *)(gcol + il));
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int i = il + e;
                        bm[e] = (bf16)((i > jl && i < q) ? exp_diff(cs_s[i], csj) * (float)gv[e]
                                                         : 0.f);
                    }
                } else {
                    bm = as_bf16x8(u32x4{0u, 0u, 0u, 0u});
                }
#pragma unroll
                for (int pt = 0; pt < PT; ++pt) {
                    const bf16x8 ad = *(const bf16x8 *)(ops_s + (pt * 16 + r) * XLD + il);
                    acc[pt] = mfma_bf16(ad, bm, acc[pt]);
                }
            }
        } else {
            for (int i0 = J * 16; i0 < q; i0 += 16) {
                const int il = i0 + grp * 4;
                const f32x4 g4 = *(const f32x4 *)(gcol + il);
                float m[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int i = il + e;
                    m[e] = (i > jl && i < q) ? exp_diff(cs_s[i], csj) * g4[e] : 0.f;
                }
#pragma unroll
                for (int pt = 0; pt < PT; ++pt) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int i = il + e;
                        const float da =
                            i < q ? to_f32(dy[(row0 + (int64_t)i * H) * P + pt * 16 + r]) : 0.f;
                        acc[pt] = mfma_f32(da, m[e], acc[pt]);
                    }
                }
            }
        }
        float xd = 0.f;
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) xd += dot4(acc[pt], xv[pt]);
        xd = sum_groups(xd);
        if (grp == 0 && vj) xdx_s[jl] = xd;
        if (vj) {
            const T *dyr = dy + (row0 + (int64_t)jl * H) * P;
            T *dxr = dx + (row0 + (int64_t)jl * H) * P;
            const float diag = to_f32(cbc[(int64_t)jl * Q + jl]) + Dh;  // M_jj + D
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) {
                const int p0 = pt * 16 + 4 * grp;
                const f32x4 d4 = load4(dyr + p0);
                dDp += dot4(d4, xv[pt]);
                store4(dxr + p0, acc[pt] + diag * d4);
            }
        }
    }
    {
        const float v0 = wave_sum(vsum), v1 = wave_sum(rh), v2 = wave_sum(dDp);
        if (lane == 0) {
            red_s[wave][0] = v0;
            red_s[wave][1] = v1;
            red_s[wave][2] = v2;
        }
    }
    __syncthreads();

    // ---------------- decay gradients ----------------
    if (wave == 0) {
        float tv[3];
#pragma unroll
        for (int k = 0; k < 3; ++k) tv[k] = red_s[0][k] + red_s[1][k] + red_s[2][k] + red_s[3][k];
        // <R_c, H_{c+1}> = e^{cs_e} <R_c, H_c> + sum_j x_j . (e^{cs_e - cs_j} R_c B_j)
        const float Tend = __expf((float)csE) * tv[1] + tv[0];
        float d[4], suf[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int k = 4 * lane + e;
            d[e] = k < q ? yy_s[k] - xdx_s[k] + (k == q - 1 ? Tend : 0.f) : 0.f;
        }
        suf[3] = d[3];
        suf[2] = d[2] + suf[3];
        suf[1] = d[1] + suf[2];
        suf[0] = d[0] + suf[1];
        float tot = suf[0];
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float o = __shfl_down(tot, off, 64);
            if (lane + off < 64) tot += o;
        }
        const float after = tot - suf[0];  // sum over the lanes above this one
        const float Ah = A[h];
        float dAp = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int k = 4 * lane + e;
            if (k < q) {
                const float dda = suf[e] + after;
                const int64_t o = (b * L + s + k) * H + h;
                ddt[o] = from_f32<T>(Ah * dda);
                dAp += to_f32(dt[o]) * dda;
            }
        }
        dAp = wave_sum(dAp);
        if (lane == 0) {
            float *pp = part + ((((int64_t)b * nc + c) * H + h) * 2);
            pp[0] = dAp;
            pp[1] = tv[2];
        }
    }
}

// ---------------------------------------------------------------------------
// The chunk's C and B rows and the blocks of M = C B^T that k_chunk_bwd_pf
// reads, written in the order its waves load them: every wave load is then
// one contiguous 1 KiB block (64 lanes x 16 bytes) instead of sixteen pieces
// of different rows.  Per (b, c, g), with T16 = Q / 16 row tiles, a lane
// l = 16 grp + r and NCF = ceil(N / 32):
//   Cf, Bf [T16][NCF][64][8]  C (B) row 16 I + r, columns 32 kc + 8 grp ...
//   Gy     [T16][8][64][8]    M row 16 I + r, columns 32 sg + 8 grp ...
//                             (blocks sg <= I / 2: the rows' causal part)
//   Gx     [T16][8][64][8]    M column 16 J + r, rows 32 sg + 8 grp ...
//                             (blocks sg >= J / 2)
//   dg     [Q]                M_jj (float32)
// Steps at or past the chunk's length read as zero.  One workgroup per
// (b, c, g, tile I): the row pieces of tile I, the Gy blocks of row tile I
// and the Gx blocks of column tile J = I, one 16 x 16 MFMA tile per wave.
// ---------------------------------------------------------------------------
template <int N>
__global__ __launch_bounds__(256) void k_bwd_frags(const bf16 *__restrict__ B,
                                                   const bf16 *__restrict__ C, bf16 *__restrict__ Gy,
                                                   bf16 *__restrict__ Gx, bf16 *__restrict__ Cf,
                                                   bf16 *__restrict__ Bf, float *__restrict__ dg,
                                                   int64_t L, int G, int Q, int nc) {
    constexpr int NCF = (N + 31) / 32;
    const int T16 = Q / 16, I = blockIdx.y;
    const int64_t bcg = blockIdx.x;
    const int g = (int)(bcg % G);
    const int64_t bc = bcg / G;
    const int c = (int)(bc % nc);
    const int64_t b = bc / nc;
    const int64_t s = (int64_t)c * Q;
    const int q = (int)min<int64_t>(Q, L - s);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int r = lane & 15, grp = lane >> 4;
    const bf16 *Cc = C + ((b * L + s) * G + g) * N, *Bc = B + ((b * L + s) * G + g) * N;
    const int64_t ld = (int64_t)G * N;
    const u32x4 z4 = {0u, 0u, 0u, 0u};
    auto row_piece = [&](const bf16 *base, int i, int k) {
        return (i < q && k < N) ? *(const u32x4 *)(base + i * ld + k) : z4;
    };
    const int64_t tile0 = bcg * T16;  // first tile of this (b, c, g)

    // row pieces of tile I
    for (int kc = wave; kc < NCF; kc += 4) {
        const int i = 16 * I + r, k = 32 * kc + 8 * grp;
        const int64_t o = (((tile0 + I) * NCF + kc) * 64 + lane) * 8;
        *(u32x4 *)(Cf + o) = row_piece(Cc, i, k);
        *(u32x4 *)(Bf + o) = row_piece(Bc, i, k);
    }
    // 16 x 16 tile of M: rows 16 ti .., columns 16 tj ..; TRANS: lane (r, grp)
    // ends with M[16 ti + 4 grp + e][16 tj + r], else M[16 ti + r][16 tj + 4 grp + e]
    auto mtile = [&](int ti, int tj, bool trans) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        const int ia = trans ? 16 * ti + r : 16 * tj + r;  // A rows: C (trans) or B
        const int ib = trans ? 16 * tj + r : 16 * ti + r;  // B rows: B (trans) or C
        const bf16 *Abase = trans ? Cc : Bc, *Bbase = trans ? Bc : Cc;
#pragma unroll
        for (int kc = 0; kc < NCF; ++kc) {
            const int k = 32 * kc + 8 * grp;
            acc = mfma_bf16(as_bf16x8(row_piece(Abase, ia, k)), as_bf16x8(row_piece(Bbase, ib, k)), acc);
        }
        return acc;
    };
    auto put4 = [&](bf16 *dst, f32x4 v) {
        bf16 o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = (bf16)v[e];
        *(u32x2 *)dst = *(const u32x2 *)o;
    };
    // a 16-step tile t inside 32-block t / 2 goes to lane group 2 (t % 2) + grp / 2,
    // elements 4 (grp % 2) ..
    auto frag_off = [&](int tile, int t) {
        return ((((tile0 + tile) * 8 + t / 2) * 64) + (2 * (t & 1) + grp / 2) * 16 + r) * 8 + 4 * (grp & 1);
    };
    // Gy: row tile I, column tiles 0 .. 2 (I / 2) + 1 (the last 32-block is the diagonal one)
    const int ny = min(2 * (I / 2) + 2, T16);
    for (int t = wave; t < ny; t += 4) put4(Gy + frag_off(I, t), mtile(I, t, false));
    // Gx: column tile J = I, row tiles 2 (I / 2) .. T16 - 1
    for (int t = 2 * (I / 2) + wave; t < T16; t += 4) {
        const f32x4 m = mtile(t, I, true);
        put4(Gx + frag_off(I, t), m);
        if (t == I) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (4 * grp + e == r) dg[bcg * Q + 16 * I + r] = m[e];
        }
    }
}

// ---------------------------------------------------------------------------
// fp32 [P][N] state -> bf16 [P][ld] in LDS (row p at rowof(p)) by NT
// threads, in two steps like TrStage: load() issues every load, write()
// converts and stores.  With DOT, write() also returns this thread's part of
// sum(src * other) over the same elements (other has src's layout).
// ---------------------------------------------------------------------------
template <int P, int N, int NT, bool DOT>
struct StateStage {
    static constexpr int NI = P * N / 8, IT = (NI + NT - 1) / NT;
    f32x4 a[IT][2], o[DOT ? IT : 1][2];
    __device__ __forceinline__ void load(const float *__restrict__ src, const float *__restrict__ other) {
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int idx = min((int)threadIdx.x + it * NT, NI - 1);
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                a[it][k] = *(const f32x4 *)(src + 8 * idx + 4 * k);
                if constexpr (DOT) o[it][k] = *(const f32x4 *)(other + 8 * idx + 4 * k);
            }
        }
    }
    template <typename RowOf = RowIdentity>
    __device__ __forceinline__ float write(bf16 *dst, int ld, RowOf rowof = RowOf{}) const {
        float acc = 0.f;
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int idx = (int)threadIdx.x + it * NT;
            if (NI % NT == 0 || idx < NI) {
                const int p = idx / (N / 8), n0 = (idx - p * (N / 8)) * 8;
                bf16x8 v;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    v[e] = (bf16)a[it][0][e];
                    v[e + 4] = (bf16)a[it][1][e];
                }
                *(bf16x8 *)(dst + rowof(p) * ld + n0) = v;
                if constexpr (DOT) acc += dot4(a[it][0], o[it][0]) + dot4(a[it][1], o[it][1]);
            }
        }
        return acc;
    }
};

// ---------------------------------------------------------------------------
// bfloat16 version of k_chunk_bwd, one workgroup per (b, c, h), that keeps
// the global loads of the next row tile in flight while the current one
// computes.  A wave's tile operands (its row of C or B, the blocks of M =
// C B^T of that row or column, 4 channels of the dy and x rows it dots with,
// the diagonal M_jj) are one register set; two sets alternate, so set k + 1
// loads while set k computes.  C, B and the M blocks come in the fragment
// order k_bwd_frags writes, one contiguous 1 KiB block per wave load.  Every
// global access goes through a buffer resource and a lane with nothing to
// load is given an offset past the resource's end, so no load or store sits
// behind a branch and the compiler's counted waits stay exact (a load behind
// a branch makes it wait for every load in flight).  The four rounds of row
// tiles are unrolled, and round R loads only the M blocks its tiles can use
// (2 R + 2 causal blocks of a row; 8 - 2 R of a column).  Same phases,
// results and outputs as k_chunk_bwd.  The launcher requires Q <= 256 and
// Q * H * P * 2 < 2^31 (every offset fits the 32-bit range).
// ---------------------------------------------------------------------------
template <int R>
using RoundC = std::integral_constant<int, R>;

template <int P, int N>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_chunk_bwd_pf(
    const bf16 *__restrict__ x, const bf16 *__restrict__ dy, const bf16 *__restrict__ dt,
    const float *__restrict__ A, const bf16 *__restrict__ Bf, const bf16 *__restrict__ Cf,
    const bf16 *__restrict__ Gy, const bf16 *__restrict__ Gx, const float *__restrict__ dg,
    const float *__restrict__ cs, const float *__restrict__ Hs, const float *__restrict__ Rs,
    const float *__restrict__ D, bf16 *__restrict__ dx, bf16 *__restrict__ ddt,
    float *__restrict__ part, int64_t L, int H, int G, int Q, int nc) {
    constexpr int PT = P / 16, NCF = (N + 31) / 32, NSEG = 8;
    const int64_t wid = xcd_remap(blockIdx.x, gridDim.x);
    const int h = (int)(wid % H);
    const int64_t bc = wid / H;
    const int c = (int)(bc % nc);
    const int64_t b = bc / nc;
    const int g = h / (H / G);
    const int64_t s = (int64_t)c * Q;
    const int q = (int)min<int64_t>(Q, L - s);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int r = lane & 15, grp = lane >> 4;

    __shared__ float cs_s[256], yy_s[256], xdx_s[256], red_s[4][3];
    const float *csc = cs + (((int64_t)b * H + h) * nc + c) * Q;
    const float cs_own = csc[min((int)threadIdx.x, Q - 1)];  // written to LDS below
    const int64_t row0 = (b * L + s) * H + h;
    const int T16Q = Q / 16;
    const int64_t tile0 = (((int64_t)b * nc + c) * G + g) * T16Q;  // first fragment tile
    const int64_t soff = (((int64_t)b * nc + c) * H + h) * (int64_t)P * N;
    const float *hp = Hs + soff, *rp = Rs + soff;
    const float Dh = D ? D[h] : 0.f;
    // byte stride between consecutive steps of one head's rows
    const uint32_t rowb = (uint32_t)H * P * 2;
    const auto rsCf = buf_rsrc(Cf + tile0 * NCF * 512, (uint32_t)T16Q * NCF * 1024);
    const auto rsBf = buf_rsrc(Bf + tile0 * NCF * 512, (uint32_t)T16Q * NCF * 1024);
    const auto rsGy = buf_rsrc(Gy + tile0 * NSEG * 512, (uint32_t)T16Q * NSEG * 1024);
    const auto rsGx = buf_rsrc(Gx + tile0 * NSEG * 512, (uint32_t)T16Q * NSEG * 1024);
    const auto rsDg = buf_rsrc(dg + tile0 * 16, (uint32_t)Q * 4);
    const auto rsDY = buf_rsrc(dy + row0 * P, (uint32_t)q * rowb);
    const auto rsX = buf_rsrc(x + row0 * P, (uint32_t)q * rowb);
    const auto rsDX = buf_rsrc(dx + row0 * P, (uint32_t)q * rowb);

    constexpr int XLD = 256 + 8, HLD = N + 8;
    __shared__ bf16 ops_s[P * XLD];
    __shared__ bf16 st_s[P * HLD];
    const u32x4 z4 = {0u, 0u, 0u, 0u};
    const int T16 = (q + 15) / 16;
    auto tile_of = [&](int round) { return 4 * round + ((round & 1) ? 3 - wave : wave); };

    struct Ops {
        u32x4 vr[NCF];
        u32x4 gs[NSEG];
        u32x2 d4[PT], x4[PT];
        float dg;
    };
    auto state_mma = [&](f32x4 *acc, const Ops &o) {
#pragma unroll
        for (int kc = 0; kc < NCF; ++kc) {
            const int kk = kc * 32 + grp * 8;
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) {
                const u32x4 av = kk < N ? *(const u32x4 *)(st_s + (pt * 16 + r) * HLD + kk) : z4;
                acc[pt] = mfma_bf16(as_bf16x8(av), as_bf16x8(o.vr[kc]), acc[pt]);
            }
        }
    };
    // A fragment block is 1 KiB: the lane's 16 bytes at lane * 16 (per-lane offset) plus the
    // block's start (wave-uniform, a scalar offset).  Blocks of a round that a tile cannot use
    // (at most one per tile) load too, unused, so the count of loads stays fixed.
    auto blk = [&](int tile, int b_, int per) { return (uint32_t)(tile * per + b_) * 1024u; };
    // Channel order in LDS: row 16 pt + 4 grp + e holds channel (P / 4) grp + 4 pt + e, so the
    // accumulators a lane ends with (tile pt, rows 4 grp + e) are the channels (P / 4) grp ..
    // (P / 4) grp + P / 4 - 1: one contiguous piece of a dy, x or dx row.
    auto prow = [](int p) { return 16 * ((p % (P / 4)) / 4) + 4 * (p / (P / 4)) + (p & 3); };
    // this lane's piece of a row at byte offset drow (zero when !valid), as 4-channel pieces
    auto row_load = [&](__amdgpu_buffer_rsrc_t rs, uint32_t drow, bool valid, u32x2(&out)[PT]) {
        const uint32_t o = drow + 2u * (P / 4) * grp;
        if constexpr (PT == 1) {
            out[0] = buf_ld8(rs, valid ? o : kBufOff);
        } else {
#pragma unroll
            for (int k2 = 0; k2 < PT / 2; ++k2) {
                const u32x4 t = buf_ld16(rs, valid ? o + 16u * k2 : kBufOff);
                out[2 * k2] = u32x2{t[0], t[1]};
                out[2 * k2 + 1] = u32x2{t[2], t[3]};
            }
        }
    };

    // ---------------- phase Y ----------------
    // round R: row tiles up to 4 R + 3, so causal blocks 0 .. 2 R + 1
    auto load_y = [&](auto RC, Ops &o) {
        constexpr int R = decltype(RC)::value, NSY = 2 * R + 2;
        const int I = tile_of(R);
        const int il = I * 16 + r;
        const bool vi = I < T16 && il < q;
        const uint32_t drow = (uint32_t)il * rowb;
        const uint32_t vo = I < T16 ? lane * 16u : kBufOff;
#pragma unroll
        for (int kc = 0; kc < NCF; ++kc) o.vr[kc] = buf_ld16s(rsCf, vo, blk(I, kc, NCF));
#pragma unroll
        for (int sg = 0; sg < NSY; ++sg) o.gs[sg] = buf_ld16s(rsGy, vo, blk(I, sg, NSEG));
        row_load(rsDY, drow, vi, o.d4);
    };
    auto comp_y = [&](auto RC, const Ops &o) {
        constexpr int R = decltype(RC)::value, NSY = 2 * R + 2;
        const int I = tile_of(R);
        const int il = I * 16 + r;
        f32x4 acc[PT];
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) acc[pt] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (I < T16) {
            const float csi = cs_s[min(il, 255)];
            state_mma(acc, o);
            const float ei = __expf(csi);
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) acc[pt] *= ei;
#pragma unroll
            for (int sg = 0; sg < NSY; ++sg) {
                if (sg * 32 <= I * 16 + 15) {
                    const int jl = sg * 32 + grp * 8;
                    const bf16x8 gv = as_bf16x8(o.gs[sg]);
                    bf16x8 bm;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int j = jl + e;
                        bm[e] = (bf16)((j < il) ? __expf(csi - cs_s[j]) * (float)gv[e] : 0.f);
                    }
#pragma unroll
                    for (int pt = 0; pt < PT; ++pt) {
                        const bf16x8 ax = *(const bf16x8 *)(ops_s + (pt * 16 + r) * XLD + jl);
                        acc[pt] = mfma_bf16(ax, bm, acc[pt]);
                    }
                }
            }
        }
        float yy = 0.f;
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) yy += dot4(acc[pt], load4((const bf16 *)&o.d4[pt]));
        yy = sum_groups(yy);
        if (grp == 0 && il < q) yy_s[il] = yy;
    };
    // x^T and H_c staged, with the first tile's loads issued before the LDS stores
    Ops o0, o1;
    {
        TrStage<256, P, 256> xst;
        StateStage<P, N, 256, false> hst;
        xst.load(rsX, rowb, q);
        hst.load(hp, nullptr);
        load_y(RoundC<0>{}, o0);
        cs_s[threadIdx.x] = cs_own;
        yy_s[threadIdx.x] = 0.f;
        xdx_s[threadIdx.x] = 0.f;
        xst.write(ops_s, XLD, prow);
        hst.write(st_s, HLD, prow);
    }
    __syncthreads();
    load_y(RoundC<1>{}, o1);
    comp_y(RoundC<0>{}, o0);
    load_y(RoundC<2>{}, o0);
    comp_y(RoundC<1>{}, o1);
    load_y(RoundC<3>{}, o1);
    comp_y(RoundC<2>{}, o0);
    // the loads of phase X's staging (dy^T, R_c, H_c) fly during the last tile
    TrStage<256, P, 256> dyst;
    StateStage<P, N, 256, true> rst;
    dyst.load(rsDY, rowb, q);
    rst.load(rp, hp);
    comp_y(RoundC<3>{}, o1);
    lds_barrier();  // every wave is done with x^T and H_c in LDS

    // ---------------- phase X ----------------
    // round R: column tiles from 4 R, so row blocks 2 R .. 7
    auto load_x = [&](auto RC, Ops &o) {
        constexpr int R = decltype(RC)::value, SX0 = 2 * R;
        const int J = tile_of(R);
        const int jl = J * 16 + r;
        const bool vj = J < T16 && jl < q;
        const uint32_t drow = (uint32_t)jl * rowb;
        const uint32_t vo = J < T16 ? lane * 16u : kBufOff;
#pragma unroll
        for (int kc = 0; kc < NCF; ++kc) o.vr[kc] = buf_ld16s(rsBf, vo, blk(J, kc, NCF));
#pragma unroll
        for (int sg = SX0; sg < NSEG; ++sg) o.gs[sg] = buf_ld16s(rsGx, vo, blk(J, sg, NSEG));
        row_load(rsDY, drow, vj, o.d4);
        row_load(rsX, drow, vj, o.x4);
        o.dg = buf_ldf(rsDg, vj ? 4u * jl : kBufOff);  // M_jj
    };
    const float csE = cs_s[q - 1];
    float vsum = 0.f, dDp = 0.f;
    auto comp_x = [&](auto RC, const Ops &o) {
        constexpr int R = decltype(RC)::value, SX0 = 2 * R;
        const int J = tile_of(R);
        const int jl = J * 16 + r;
        const bool vj = jl < q;
        f32x4 acc[PT], xv[PT];
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) {
            acc[pt] = f32x4{0.f, 0.f, 0.f, 0.f};
            xv[pt] = load4((const bf16 *)&o.x4[pt]);
        }
        if (J < T16) {
            const float csj = cs_s[min(jl, 255)];
            state_mma(acc, o);
            const float wj = __expf(csE - csj);
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) {
                acc[pt] *= wj;
                vsum += dot4(acc[pt], xv[pt]);
            }
            const int ilo = (J * 16) & ~31;
#pragma unroll
            for (int sg = SX0; sg < NSEG; ++sg) {
                const int i0 = sg * 32;
                if (i0 >= ilo && i0 < q) {
                    const int il = i0 + grp * 8;
                    const bf16x8 gv = as_bf16x8(o.gs[sg]);
                    bf16x8 bm;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int i = il + e;
                        bm[e] = (bf16)((i > jl && i < q) ? __expf(cs_s[i] - csj) * (float)gv[e] : 0.f);
                    }
#pragma unroll
                    for (int pt = 0; pt < PT; ++pt) {
                        const bf16x8 ad = *(const bf16x8 *)(ops_s + (pt * 16 + r) * XLD + il);
                        acc[pt] = mfma_bf16(ad, bm, acc[pt]);
                    }
                }
            }
        }
        float xd = 0.f;
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) xd += dot4(acc[pt], xv[pt]);
        xd = sum_groups(xd);
        if (grp == 0 && vj) xdx_s[jl] = xd;
        const float diag = o.dg + Dh;  // M_jj + D
        const uint32_t drow = (uint32_t)jl * rowb + 2u * (P / 4) * grp;
        u32x2 packed[PT];
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) {
            const f32x4 d4 = load4((const bf16 *)&o.d4[pt]);
            dDp += dot4(d4, xv[pt]);
            const f32x4 v = acc[pt] + diag * d4;
            bf16 ob[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) ob[e] = (bf16)v[e];
            packed[pt] = *(const u32x2 *)ob;
        }
        if constexpr (PT == 1) {
            buf_st8(packed[0], rsDX, vj ? drow : kBufOff);
        } else {
#pragma unroll
            for (int k2 = 0; k2 < PT / 2; ++k2)
                buf_st16(u32x4{packed[2 * k2][0], packed[2 * k2][1], packed[2 * k2 + 1][0],
                               packed[2 * k2 + 1][1]},
                         rsDX, vj ? drow + 16u * k2 : kBufOff);
        }
    };
    load_x(RoundC<0>{}, o0);
    dyst.write(ops_s, XLD, prow);
    {
        // <R_c, H_c>, reduced here so that the products are not kept to the end
        const float rh = wave_sum(rst.write(st_s, HLD, prow));
        if (lane == 0) red_s[wave][1] = rh;
    }
    __syncthreads();
    // the step sizes of the chunk for the decay gradients (wave 0, lane l: steps 4 l ..)
    const auto rsDT = buf_rsrc(dt + (b * L + s) * H + h, (uint32_t)q * H * 2);
    const auto rsDDT = buf_rsrc(ddt + (b * L + s) * H + h, (uint32_t)q * H * 2);
    uint16_t dtv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int k = 4 * lane + e;
        dtv[e] = buf_ld2(rsDT, (wave == 0 && k < q) ? (uint32_t)(k * H * 2) : kBufOff);
    }
    load_x(RoundC<1>{}, o1);
    comp_x(RoundC<0>{}, o0);
    load_x(RoundC<2>{}, o0);
    comp_x(RoundC<1>{}, o1);
    load_x(RoundC<3>{}, o1);
    comp_x(RoundC<2>{}, o0);
    comp_x(RoundC<3>{}, o1);
    {
        const float v0 = wave_sum(vsum), v2 = wave_sum(dDp);
        if (lane == 0) {
            red_s[wave][0] = v0;
            red_s[wave][2] = v2;
        }
    }
    __syncthreads();

    // ---------------- decay gradients ----------------
    if (wave == 0) {
        float tv[3];
#pragma unroll
        for (int k = 0; k < 3; ++k) tv[k] = red_s[0][k] + red_s[1][k] + red_s[2][k] + red_s[3][k];
        const float Tend = __expf(csE) * tv[1] + tv[0];
        float d[4], suf[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int k = 4 * lane + e;
            d[e] = k < q ? yy_s[k] - xdx_s[k] + (k == q - 1 ? Tend : 0.f) : 0.f;
        }
        suf[3] = d[3];
        suf[2] = d[2] + suf[3];
        suf[1] = d[1] + suf[2];
        suf[0] = d[0] + suf[1];
        float tot = suf[0];
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float o = __shfl_down(tot, off, 64);
            if (lane + off < 64) tot += o;
        }
        const float after = tot - suf[0];
        const float Ah = A[h];
        float dAp = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int k = 4 * lane + e;
            const float dda = suf[e] + after;
            buf_st2(__builtin_bit_cast(uint16_t, (bf16)(Ah * dda)), rsDDT,
                    k < q ? (uint32_t)(k * H * 2) : kBufOff);
            dAp += k < q ? (float)__builtin_bit_cast(bf16, dtv[e]) * dda : 0.f;
        }
        dAp = wave_sum(dAp);
        if (lane == 0) {
            float *pp = part + ((((int64_t)b * nc + c) * H + h) * 2);
            pp[0] = dAp;
            pp[1] = tv[2];
        }
    }
}

// ---------------------------------------------------------------------------
// Per (b, c, g, 64-row tile): sums over the heads of group g of
//   dCB[i][j] = exp(cs_i - cs_j) (dy_i . x_j)                  (j <= i)
//   dCs[i][n] = exp(cs_i) sum_p dy_i[p] H_c[p][n]
//   dBs[j][n] = exp(cs_e - cs_j) sum_p x_j[p] R_c[p][n]
// Each wave owns 16 rows and keeps its accumulators in registers across the
// head loop; the row operands (dy_i, x_i) are 16-byte fragments straight
// from global memory, the column operands (x_j, a state column) likewise.
// dCB is written in both orientations (dcb[i][j], dcbT[j][i]); tiles above
// the diagonal are not written.
// ---------------------------------------------------------------------------
template <typename T, int P, int N, typename CsT>
__global__ __launch_bounds__(256) void k_group_bwd(
    const T *__restrict__ x, const T *__restrict__ dy, const CsT *__restrict__ cs,
    const float *__restrict__ Hs, const float *__restrict__ Rs, float *__restrict__ dcb,
    float *__restrict__ dcbT, float *__restrict__ dCs, float *__restrict__ dBs, int64_t L, int H,
    int G, int Q, int nc) {
    constexpr int KPL = Frag<T>::KPL, KSTEP = Frag<T>::KSTEP;
    constexpr int KS = (P + KSTEP - 1) / KSTEP, NT = N / 16;
    const int ntr = (Q + 63) / 64;
    const int64_t work = xcd_remap(blockIdx.x, gridDim.x);
    const int tile = (int)(work % ntr);
    const int64_t bcg = work / ntr;
    const int g = (int)(bcg % G);
    const int64_t bc = bcg / G;
    const int c = (int)(bc % nc);
    const int64_t b = bc / nc;
    const int64_t s = (int64_t)c * Q;
    const int q = (int)min<int64_t>(Q, L - s);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int r = lane & 15, grp = lane >> 4;
    const int i0 = tile * 64 + wave * 16;
    if (i0 >= q) return;  // no barriers below
    const int Ti = i0 / 16;
    const int ia = i0 + r;  // this lane's row in the row-operand fragments
    const bool va = ia < q;

    f32x4 acb[16], adc[NT], adb[NT];
#pragma unroll
    for (int J = 0; J < 16; ++J) acb[J] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < NT; ++t) adc[t] = adb[t] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int hpg = H / G;
    const u32x4 z = {0u, 0u, 0u, 0u};
    for (int hh = 0; hh < hpg; ++hh) {
        const int h = g * hpg + hh;
        const CsT *csh = cs + (((int64_t)b * H + h) * nc + c) * Q;
        const CsT csE = csh[q - 1];
        CsT csr[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) csr[e] = csh[min(i0 + 4 * grp + e, Q - 1)];
        const CsT csa = csh[min(ia, Q - 1)];
        const float ea = __expf((float)csa), wa = exp_diff(csE, csa);
        const int64_t rowA = (b * L + s + ia) * H + h;
        u32x4 fdy[KS], fdye[KS], fxw[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int kk = ks * KSTEP + grp * KPL;
            const bool ok = va && kk < P;
            const u32x4 dv = ok ? *(const u32x4 *)(dy + rowA * P + kk) : z;
            const u32x4 xv = ok ? *(const u32x4 *)(x + rowA * P + kk) : z;
            fdy[ks] = dv;
            fdye[ks] = frag_scale<T>(dv, ea);
            fxw[ks] = frag_scale<T>(xv, wa);
        }
        // masked dy_i . x_j, j-tiles up to the diagonal
#pragma unroll
        for (int J = 0; J < 16; ++J) {
            if (J <= Ti) {
                const int jr = J * 16 + r;
                const bool vj = jr < q;
                const int64_t rowB = (b * L + s + jr) * H + h;
                f32x4 t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const int kk = ks * KSTEP + grp * KPL;
                    const u32x4 bx = (vj && kk < P) ? *(const u32x4 *)(x + rowB * P + kk) : z;
                    t = mma16<T>(fdy[ks], bx, t);
                }
                const CsT csj = csh[min(jr, Q - 1)];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int i = i0 + 4 * grp + e;
                    acb[J][e] += (jr <= i && i < q) ? exp_diff(csr[e], csj) * t[e] : 0.f;
                }
            }
        }
        // state terms: column operand = state column n, KPL consecutive p
        const int64_t soff = (((int64_t)b * nc + c) * H + h) * (int64_t)P * N;
        const float *hp = Hs + soff, *rp = Rs + soff;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const int n = t * 16 + r;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int kk = ks * KSTEP + grp * KPL;
                const u32x4 bh = kk < P ? frag_from_f32_col<T>(hp + (int64_t)kk * N + n, N) : z;
                const u32x4 br = kk < P ? frag_from_f32_col<T>(rp + (int64_t)kk * N + n, N) : z;
                adc[t] = mma16<T>(fdye[ks], bh, adc[t]);
                adb[t] = mma16<T>(fxw[ks], br, adb[t]);
            }
        }
    }

    const int64_t cboff = bcg * (int64_t)Q * Q;
#pragma unroll
    for (int J = 0; J < 16; ++J) {
        if (J <= Ti) {
            const int jr = J * 16 + r;
#pragma unroll
            for (int e = 0; e < 4; ++e) dcb[cboff + (int64_t)(i0 + 4 * grp + e) * Q + jr] = acb[J][e];
            *(f32x4 *)(dcbT + cboff + (int64_t)jr * Q + i0 + 4 * grp) = acb[J];
        }
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const int n = t * 16 + r;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = i0 + 4 * grp + e;
            if (i < q) {
                const int64_t o = ((b * L + s + i) * G + g) * N + n;
                dCs[o] = adc[t][e];
                dBs[o] = adb[t][e];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// bfloat16: dCB[i][j] = sum_h exp(cs_i - cs_j) (dy_i . x_j) alone, one
// workgroup per (b, c, g, 64 x 64 block on or below the diagonal); wave
// (wr, wc) owns the 32 x 32 piece at rows 32 wr, columns 32 wc of the block
// (the piece wholly above the diagonal of a diagonal block is skipped).  The
// head loop keeps only this piece's accumulators, with the next head's row
// and column fragments and decay prefix values loaded while the current head
// computes.  Writes dcb[i][j] and dcbT[j][i] for the 16 x 16 tiles on or
// below the diagonal (the others are never read).
// ---------------------------------------------------------------------------
template <int P>
__global__ __launch_bounds__(256) void k_group_dcb(const bf16 *__restrict__ x,
                                                   const bf16 *__restrict__ dy,
                                                   const float *__restrict__ cs,
                                                   float *__restrict__ dcb,
                                                   float *__restrict__ dcbT, int64_t L, int H,
                                                   int G, int Q, int nc) {
    constexpr int KS = P / 32 > 0 ? P / 32 : 1;
    const int nbk = (Q + 63) / 64, npair = nbk * (nbk + 1) / 2;
    const int64_t work = xcd_remap(blockIdx.x, gridDim.x);
    const int pair = (int)(work % npair);
    const int64_t bcg = work / npair;
    int IB = (int)((sqrtf(8.f * pair + 1.f) - 1.f) * 0.5f);
    while ((IB + 1) * (IB + 2) / 2 <= pair) ++IB;
    while (IB * (IB + 1) / 2 > pair) --IB;
    const int JB = pair - IB * (IB + 1) / 2;
    const int g = (int)(bcg % G);
    const int64_t bc = bcg / G;
    const int c = (int)(bc % nc);
    const int64_t b = bc / nc;
    const int64_t s = (int64_t)c * Q;
    const int q = (int)min<int64_t>(Q, L - s);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int r = lane & 15, grp = lane >> 4;
    const int wr = wave >> 1, wc = wave & 1;
    const int i0 = IB * 64 + 32 * wr, j0 = JB * 64 + 32 * wc;
    if (i0 >= q || j0 > i0 + 31) return;  // nothing of this piece is read; no barriers below
    const u32x4 z = {0u, 0u, 0u, 0u};
    const int hpg = H / G;

    f32x4 acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int bb = 0; bb < 2; ++bb) acc[a][bb] = f32x4{0.f, 0.f, 0.f, 0.f};

    u32x4 pa[2][KS], pb[2][KS];
    float pci[2][4], pcj[2];
    auto load = [&](int h) {
        const float *csh = cs + (((int64_t)b * H + h) * nc + c) * Q;
#pragma unroll
        for (int a = 0; a < 2; ++a) {
            const int ir = i0 + 16 * a + r, jr = j0 + 16 * a + r;
            const int64_t ri = (b * L + s + ir) * H + h, rj = (b * L + s + jr) * H + h;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int kk = ks * 32 + grp * 8;
                pa[a][ks] = (ir < q && kk < P) ? *(const u32x4 *)(dy + ri * P + kk) : z;
                pb[a][ks] = (jr < q && kk < P) ? *(const u32x4 *)(x + rj * P + kk) : z;
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) pci[a][e] = csh[min(i0 + 16 * a + 4 * grp + e, Q - 1)];
            pcj[a] = csh[min(jr, Q - 1)];
        }
    };
    load(g * hpg);
    for (int hh = 0; hh < hpg; ++hh) {
        u32x4 fa[2][KS], fb[2][KS];
        float ci[2][4], cj[2];
#pragma unroll
        for (int a = 0; a < 2; ++a) {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                fa[a][ks] = pa[a][ks];
                fb[a][ks] = pb[a][ks];
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) ci[a][e] = pci[a][e];
            cj[a] = pcj[a];
        }
        if (hh + 1 < hpg) load(g * hpg + hh + 1);
#pragma unroll
        for (int a = 0; a < 2; ++a) {
#pragma unroll
            for (int bb = 0; bb < 2; ++bb) {
                f32x4 t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    t = mfma_bf16(as_bf16x8(fa[a][ks]), as_bf16x8(fb[bb][ks]), t);
                const int j = j0 + 16 * bb + r;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int i = i0 + 16 * a + 4 * grp + e;
                    acc[a][bb][e] += (j <= i && i < q) ? __expf(ci[a][e] - cj[bb]) * t[e] : 0.f;
                }
            }
        }
    }
    const int64_t cboff = bcg * (int64_t)Q * Q;
#pragma unroll
    for (int a = 0; a < 2; ++a) {
#pragma unroll
        for (int bb = 0; bb < 2; ++bb) {
            const int it = i0 + 16 * a, jt = j0 + 16 * bb;
            if (jt > it || it >= Q) continue;  // tile above the diagonal or past the chunk
            const int j = jt + r;
#pragma unroll
            for (int e = 0; e < 4; ++e) dcb[cboff + (int64_t)(it + 4 * grp + e) * Q + j] = acc[a][bb][e];
            *(f32x4 *)(dcbT + cboff + (int64_t)j * Q + it + 4 * grp) = acc[a][bb];
        }
    }
}

// ---------------------------------------------------------------------------
// bfloat16 dCB for P in {32, 64}, one workgroup per (b, c, g, 64-row block
// IB): the block pairs (IB, JB), JB <= IB, are split over the waves (two
// waves per pair for P = 64, each with half its rows) and the head loop runs
// once for all of them, so dy rows of block IB and x rows of blocks 0..IB
// are loaded once per head for up to four pairs (instead of once per
// pair).  Per head the waves copy those rows and the chunk's decay
// prefix straight into a slot of a three-slot LDS ring with direct
// global-to-LDS loads (no registers in flight), two heads ahead; each wave
// waits only for its own copies of the head it is about to use (a counted
// vmcnt: every wave issues the same number of copies per head, all lanes
// active) and one barrier per head publishes the slot and frees the oldest.
// Rows are 16-byte chunks stored at chunk ^ (row & (chunks per row - 1)),
// so the MFMA fragment reads of 16 rows hit distinct banks; rows past the
// chunk end are copies of its last row (their products are never stored).
// ---------------------------------------------------------------------------
namespace {

// s_waitcnt with vmcnt = N (lgkmcnt and expcnt at their maxima)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70 | 0xF00);
}

constexpr int kDcbSlots = 3;
template <int P>
struct DcbRing {
    static constexpr int ROWB = P * 2;               // bytes per row
    static constexpr int CPR = ROWB / 16;            // 16-byte chunks per row
    static constexpr int BLK = 64 * ROWB;            // bytes per 64-row block
    static constexpr int IPB = BLK / 1024;           // wave copies per block
    static constexpr int SLOT = 5 * BLK + 1024;      // dy block + up to 4 x blocks + cs
};

// NW waves: wave w computes rows 16 a, a in [NA * (w % (NW / 4)), + NA), of
// the pair (IB, JB = w / (NW / 4)), NA = 16 / NW.
template <int P>
constexpr int dcb_waves() { return P == 64 ? 8 : 4; }

template <int P, int IB>
__device__ __forceinline__ void group_dcb_rb_body(unsigned char (*ring)[DcbRing<P>::SLOT],
                                                  const bf16 *__restrict__ x, const bf16 *__restrict__ dy,
                                                  const float *__restrict__ cs, float *__restrict__ dcb,
                                                  float *__restrict__ dcbT, int64_t L, int H, int G, int Q,
                                                  int nc, int64_t bcg) {
    using R = DcbRing<P>;
    constexpr int NW = dcb_waves<P>(), WPP = NW / 4, NA = 4 / WPP;
    constexpr int NBLK = IB + 2;                      // dy block IB, x blocks 0..IB
    constexpr int NBI = NBLK * R::IPB;                // block copies per head
    static_assert(NBI % NW == 0, "block copies split evenly over the waves");
    constexpr int NIW = NBI / NW + 1;                 // copies per wave per head (+ its share of cs)
    constexpr int CSL = 64 / NW;                      // lanes per cs share (16 bytes each)
    constexpr int KS = P / 32;
    const int g = (int)(bcg % G);
    const int64_t bc = bcg / G;
    const int c = (int)(bc % nc);
    const int64_t b = bc / nc;
    const int64_t s = (int64_t)c * Q;
    const int q = (int)min<int64_t>(Q, L - s);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int r = lane & 15, grp = lane >> 4;
    const int hpg = H / G, h0 = g * hpg;
    const int JB = wave / WPP, a0 = NA * (wave % WPP);
    const bool active = JB <= IB;                     // computes rows a0.. of pair (IB, JB)

    auto issue = [&](int hh, int slot) {
        const int h = h0 + hh;
        unsigned char *base = ring[slot];
#pragma unroll
        for (int k0 = 0; k0 < NBI; k0 += NW) {
            const int k = k0 + wave;
            const int blk = k / R::IPB, sub = k % R::IPB;
            constexpr int RPI = 1024 / R::ROWB;       // rows per copy
            const int row = sub * RPI + lane / R::CPR;
            const int chunk = (lane % R::CPR) ^ (row & (R::CPR - 1));
            const int grow = min((blk == 0 ? IB : blk - 1) * 64 + row, q - 1);
            const bf16 *src = (blk == 0 ? dy : x) + ((b * L + s + grow) * H + h) * P + chunk * 8;
            copy16_to_lds(src, base + blk * R::BLK + sub * 1024);
        }
        // decay prefix: wave w copies floats 4 CSL w .. + 4 CSL - 1 with lanes 0..CSL-1
        // (16 bytes each); the copy always has active lanes, so it counts once per
        // wave like the block copies
        if (lane < CSL) {
            const int f = min(4 * (CSL * wave + lane), Q - 4);
            copy16_to_lds(cs + (((int64_t)b * H + h) * nc + c) * Q + f,
                          base + 5 * R::BLK + wave * (16 * CSL));
        }
    };

    f32x4 acc[NA][4];
#pragma unroll
    for (int a = 0; a < NA; ++a)
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) acc[a][bb] = f32x4{0.f, 0.f, 0.f, 0.f};

    issue(0, 0);
    if (hpg > 1) issue(1, 1);
    constexpr float kL2e = 1.4426950408889634f;
    for (int hh = 0; hh < hpg; ++hh) {
        const int slot = hh % kDcbSlots;
        // this wave's copies of head hh are done once at most the next head's are in flight
        if (hh + 1 < hpg) wait_vmcnt<NIW>(); else wait_vmcnt<0>();
        __atomic_signal_fence(__ATOMIC_SEQ_CST);  // keep LDS accesses on their side of the barrier
        __builtin_amdgcn_s_barrier();
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        if (hh + 2 < hpg) issue(hh + 2, (hh + 2) % kDcbSlots);
        if (!active) continue;
        const unsigned char *base = ring[slot];
        const bf16 *dys = (const bf16 *)base;
        const bf16 *xsb = (const bf16 *)(base + (1 + JB) * R::BLK);
        const float *css = (const float *)(base + 5 * R::BLK);
        float cj[4];
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) cj[bb] = css[64 * JB + 16 * bb + r] * kL2e;
        bf16x8 fb[4][KS];
#pragma unroll
        for (int bb = 0; bb < 4; ++bb)
#pragma unroll
            for (int kc = 0; kc < KS; ++kc) {
                const int row = 16 * bb + r, ch = (4 * kc + grp) ^ (row & (R::CPR - 1));
                fb[bb][kc] = *(const bf16x8 *)(xsb + row * P + ch * 8);
            }
#pragma unroll
        for (int ai = 0; ai < NA; ++ai) {
            const int a = a0 + ai;
            bf16x8 fa[KS];
#pragma unroll
            for (int kc = 0; kc < KS; ++kc) {
                const int row = 16 * a + r, ch = (4 * kc + grp) ^ (row & (R::CPR - 1));
                fa[kc] = *(const bf16x8 *)(dys + row * P + ch * 8);
            }
            float ci[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) ci[e] = css[64 * IB + 16 * a + 4 * grp + e] * kL2e;
            // all four products first, then the masks (independent work covers the MFMA latency)
            f32x4 t[4];
#pragma unroll
            for (int bb = 0; bb < 4; ++bb) {
                t[bb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kc = 0; kc < KS; ++kc) t[bb] = mfma_bf16(fa[kc], fb[bb][kc], t[bb]);
            }
#pragma unroll
            for (int bb = 0; bb < 4; ++bb) {
                const int j = 64 * JB + 16 * bb + r;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int i = 64 * IB + 16 * a + 4 * grp + e;
                    const bool keep = (IB > JB || j <= i) && i < q;
                    acc[ai][bb][e] += keep ? __builtin_amdgcn_exp2f(ci[e] - cj[bb]) * t[bb][e] : 0.f;
                }
            }
        }
    }
    if (!active) return;
    const int64_t cboff = bcg * (int64_t)Q * Q;
#pragma unroll
    for (int ai = 0; ai < NA; ++ai) {
        const int a = a0 + ai;
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
            const int it = 64 * IB + 16 * a, jt = 64 * JB + 16 * bb;
            if (jt > it || it >= Q) continue;  // tile above the diagonal or past the chunk
            const int j = jt + r;
#pragma unroll
            for (int e = 0; e < 4; ++e) dcb[cboff + (int64_t)(it + 4 * grp + e) * Q + j] = acc[ai][bb][e];
            *(f32x4 *)(dcbT + cboff + (int64_t)j * Q + it + 4 * grp) = acc[ai][bb];
        }
    }
}

}  // namespace

template <int P>
__global__ __launch_bounds__(64 * dcb_waves<P>()) void k_group_dcb_rb(const bf16 *__restrict__ x, const bf16 *__restrict__ dy,
                                                      const float *__restrict__ cs, float *__restrict__ dcb,
                                                      float *__restrict__ dcbT, int64_t L, int H, int G, int Q,
                                                      int nc) {
    __shared__ __attribute__((aligned(16))) unsigned char ring[kDcbSlots][DcbRing<P>::SLOT];
    const int nbk = (Q + 63) / 64;
    // the nbk row blocks of one (b, c, g) are neighbours, so they share an XCD's L2
    const int64_t work = xcd_remap(blockIdx.x, gridDim.x);
    const int IB = (int)(work % nbk);
    const int64_t bcg = work / nbk;
    switch (IB) {
    case 0: group_dcb_rb_body<P, 0>(ring, x, dy, cs, dcb, dcbT, L, H, G, Q, nc, bcg); break;
    case 1: group_dcb_rb_body<P, 1>(ring, x, dy, cs, dcb, dcbT, L, H, G, Q, nc, bcg); break;
    case 2: group_dcb_rb_body<P, 2>(ring, x, dy, cs, dcb, dcbT, L, H, G, Q, nc, bcg); break;
    default: group_dcb_rb_body<P, 3>(ring, x, dy, cs, dcb, dcbT, L, H, G, Q, nc, bcg); break;
    }
}

// ---------------------------------------------------------------------------
// bfloat16: the state terms alone, one workgroup of NW waves per (b, c, g,
// which, block of 16 NW rows): which = 0: dCs[i] = sum_h exp(cs_i) dy_i^T
// H_c; which = 1: dBs[j] = sum_h exp(cs_e - cs_j) x_j^T R_c.  Each wave owns
// 16 rows and keeps their accumulators across the head loop.  Per head the
// state is converted to bf16 once into LDS, row-major with the pair swizzle,
// and read as MFMA fragments with transposing reads (two LDS buffers, one
// barrier per head).  Every global load of a head (state, row fragments,
// decay prefix) is issued two heads ahead and none sits behind a branch (the
// head index is clamped), so the compiler's counted waits keep them in
// flight.
// ---------------------------------------------------------------------------
template <int P, int N, int NW>
__global__ __launch_bounds__(64 * NW) void k_group_state(
    const bf16 *__restrict__ x, const bf16 *__restrict__ dy, const float *__restrict__ cs,
    const float *__restrict__ Hs, const float *__restrict__ Rs, float *__restrict__ dCs,
    float *__restrict__ dBs, int64_t L, int H, int G, int Q, int nc) {
    constexpr int NTH = 64 * NW, ROWS = 16 * NW;
    constexpr int KS = P / 32 > 0 ? P / 32 : 1, NT = N / 16;
    constexpr int PR = P < 32 ? 32 : P;       // state rows in LDS (a fragment spans 32)
    constexpr int ROWB = N * 2;               // bytes of one bf16 state row
    constexpr int NCH = P * N / 8;            // 16-byte chunks of one bf16 state
    constexpr int CPT = (NCH + NTH - 1) / NTH;
    const int ntr = (Q + ROWS - 1) / ROWS;
    const int64_t work = xcd_remap(blockIdx.x, gridDim.x);
    const int tile = (int)(work % ntr);
    const int which = (int)((work / ntr) % 2);
    const int64_t bcg = work / (2 * ntr);
    const int g = (int)(bcg % G);
    const int64_t bc = bcg / G;
    const int c = (int)(bc % nc);
    const int64_t b = bc / nc;
    const int64_t s = (int64_t)c * Q;
    const int q = (int)min<int64_t>(Q, L - s);
    if (tile * ROWS >= q) return;  // the whole workgroup: no barrier is reached
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int r = lane & 15, grp = lane >> 4;
    const int i0 = tile * ROWS + wave * 16;
    const int ia = i0 + r, iac = min(ia, q - 1);
    const bf16 *rowsrc = which == 0 ? dy : x;
    const float *St = which == 0 ? Hs : Rs;

    __shared__ __align__(16) unsigned char st_s[2][PR * ROWB];
    if constexpr (PR > P) {
        // rows P .. PR - 1 meet zero row fragments, but must not hold NaN patterns
        for (int k = tid; k < 2 * (PR - P) * ROWB / 16; k += NTH) {
            const int bfr = k / ((PR - P) * ROWB / 16), o = k % ((PR - P) * ROWB / 16);
            *(u32x4 *)(st_s[bfr] + P * ROWB + 16 * o) = u32x4{0u, 0u, 0u, 0u};
        }
    }
    f32x4 acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int hpg = H / G, hbase = g * hpg;

    struct HeadRegs {
        f32x4 st[CPT][2];
        u32x4 row[KS];
        float ca, ce;
    };
    auto load = [&](int hh, HeadRegs &R) {
        const int h = hbase + min(hh, hpg - 1);
        const float *src = St + (((int64_t)b * nc + c) * H + h) * (int64_t)P * N;
#pragma unroll
        for (int u = 0; u < CPT; ++u) {
            const int idx = min(tid + NTH * u, NCH - 1);
            R.st[u][0] = *(const f32x4 *)(src + 8 * idx);
            R.st[u][1] = *(const f32x4 *)(src + 8 * idx + 4);
        }
        const float *csh = cs + (((int64_t)b * H + h) * nc + c) * Q;
        R.ca = csh[min(ia, Q - 1)];
        R.ce = csh[q - 1];
        const bf16 *rp = rowsrc + ((b * L + s + iac) * H + h) * (int64_t)P;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) R.row[ks] = *(const u32x4 *)(rp + min(ks * 32 + grp * 8, P - 8));
    };
    // live = false (the odd head past the group's end): the same steps, adding zero
    auto head = [&](const HeadRegs &R, int buf, bool live) {
        unsigned char *sb = st_s[buf];
#pragma unroll
        for (int u = 0; u < CPT; ++u) {
            const int idx = tid + NTH * u;
            if (NCH % NTH == 0 || idx < NCH) {
                const int p = idx / (N / 8), ch = idx % (N / 8);
                bf16x8 v;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    v[e] = (bf16)R.st[u][0][e];
                    v[e + 4] = (bf16)R.st[u][1][e];
                }
                *(bf16x8 *)(sb + p * ROWB + tr_chunk_slot<ROWB>(p, ch) * 16) = v;
            }
        }
        // (a weight of zero, not a branch: the compiler would move the row loads into one)
        const float pw = (which == 0 ? __expf(R.ca) : __expf(R.ce - R.ca)) * (live ? 1.f : 0.f);
        u32x4 fr[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            fr[ks] = ks * 32 + grp * 8 < P ? frag_scale<bf16>(R.row[ks], pw) : u32x4{0u, 0u, 0u, 0u};
        lds_barrier();  // this head's state is in LDS for every wave
#pragma unroll
        for (int t = 0; t < NT; ++t) {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                acc[t] = mfma_bf16(as_bf16x8(fr[ks]), frag_tr<ROWB>(sb, ks * 32, t * 16, lane), acc[t]);
        }
    };
    // Buffer hh & 1 is rewritten at head hh + 2, after the barrier of head hh + 1,
    // which every wave reaches only once its reads of head hh are done.  No head
    // sits behind a branch (the compiler would move its loads there).
    // sched_barrier: the scheduler keeps each group of loads where it is written.
    HeadRegs R0, R1;
    load(0, R0);
    load(1, R1);
    __builtin_amdgcn_sched_barrier(0);
    for (int hh = 0; hh < hpg; hh += 2) {
        head(R0, 0, true);
        __builtin_amdgcn_sched_barrier(0);
        load(hh + 2, R0);
        __builtin_amdgcn_sched_barrier(0);
        head(R1, 1, hh + 1 < hpg);
        __builtin_amdgcn_sched_barrier(0);
        load(hh + 3, R1);
        __builtin_amdgcn_sched_barrier(0);
    }
    if (i0 >= q) return;
    float *out = which == 0 ? dCs : dBs;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const int n = t * 16 + r;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = i0 + 4 * grp + e;
            if (i < q) out[((b * L + s + i) * G + g) * N + n] = acc[t][e];
        }
    }
}

// ---------------------------------------------------------------------------
// Per (b, c, g, which, 64-row block): which = 0: dC[i] = dCs[i] +
// sum_{j<=i} dCB[i][j] B_j; which = 1: dB[j] = dBs[j] + sum_{i>=j} dCB[i][j]
// C_i.  float32 MFMA (16x16x4).  The column operand (B or C rows) is staged
// 32 steps at a time in LDS as float32 (16-byte loads, shared by the four
// waves); wave w owns rows 16 w .. 16 w + 15 of the block and all N columns,
// and reads its dCB row segments (4 consecutive float32 per lane) straight
// from global memory.  dCB tiles above the diagonal are never written, so
// each wave stops (which 0) or starts (which 1) at its own diagonal tile.
// ---------------------------------------------------------------------------
template <typename T, int N>
__global__ __launch_bounds__(256) void k_group_combine(
    const T *__restrict__ B, const T *__restrict__ C, const float *__restrict__ dcb,
    const float *__restrict__ dcbT, const float *__restrict__ dCs, const float *__restrict__ dBs,
    T *__restrict__ dB, T *__restrict__ dC, int64_t L, int G, int Q, int nc) {
    constexpr int NT = N / 16, SK = 32, VLD = N + 4;
    const int NB64 = (Q + 63) / 64;
    const int64_t work = xcd_remap(blockIdx.x, gridDim.x);
    const int blk = (int)(work % NB64);
    const int which = (int)((work / NB64) % 2);
    const int64_t bcg = work / (2 * NB64);
    const int g = (int)(bcg % G);
    const int64_t bc = bcg / G;
    const int c = (int)(bc % nc);
    const int64_t b = bc / nc;
    const int64_t s = (int64_t)c * Q;
    const int q = (int)min<int64_t>(Q, L - s);
    if (blk * 64 >= q) return;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int r = lane & 15, grp = lane >> 4;
    const int t0 = blk * 64 + wave * 16;          // this wave's first row
    const bool wv = t0 < q;
    const int64_t cboff = bcg * (int64_t)Q * Q;
    // (row clamped: a wave past q still loads, unused, from inside this block)
    const float *arow = (which == 0 ? dcb : dcbT) + cboff + (int64_t)min(t0 + r, Q - 1) * Q;
    const T *V = (which == 0 ? B : C) + ((b * L + s) * G + g) * N;
    const int q16 = (q + 15) & ~15;
    // this wave's k range, and the workgroup's (the union over its waves)
    const int k_lo = which == 0 ? 0 : t0, k_hi = which == 0 ? t0 + 16 : q16;
    const int g_lo = which == 0 ? 0 : blk * 64;
    const int g_hi = which == 0 ? min(blk * 64 + 64, q16) : q16;
    // V rows k0 .. k0 + 31 as float32 in one of two LDS buffers; the next
    // slab's rows (and this wave's C B^T pieces) load into registers while the
    // current one multiplies.  Loads are unconditional (row indices clamped,
    // values past q zeroed after the load), so the compiler's counted waits
    // keep them in flight.
    __shared__ float vs[2][SK * VLD];
    constexpr int VPT = (SK * N / 8 + 255) / 256;  // 8-value pieces per thread per slab
    struct VRegs {
        u32x4 v[VPT][sizeof(T) == 2 ? 1 : 2];
    };
    auto load_v = [&](int k0, VRegs &R) {
#pragma unroll
        for (int u = 0; u < VPT; ++u) {
            const int idx = min((int)threadIdx.x + 256 * u, SK * N / 8 - 1);
            const int kr = idx / (N / 8), c8 = (idx % (N / 8)) * 8;
            const T *src = V + (int64_t)min(k0 + kr, q - 1) * G * N + c8;
            R.v[u][0] = *(const u32x4 *)src;
            if constexpr (sizeof(T) == 4) R.v[u][1] = *(const u32x4 *)(src + 4);
        }
    };
    auto write_v = [&](int k0, const VRegs &R, float *dst) {
#pragma unroll
        for (int u = 0; u < VPT; ++u) {
            const int idx = (int)threadIdx.x + 256 * u;
            if ((SK * N / 8) % 256 == 0 || idx < SK * N / 8) {
                const int kr = idx / (N / 8), c8 = (idx % (N / 8)) * 8;
                const bool ok = k0 + kr < q;
                float f[8];
                if constexpr (sizeof(T) == 2) {
                    const bf16x8 t = as_bf16x8(R.v[u][0]);
#pragma unroll
                    for (int e = 0; e < 8; ++e) f[e] = ok ? (float)t[e] : 0.f;
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        f[e] = ok ? __builtin_bit_cast(float, (uint32_t)R.v[u][0][e]) : 0.f;
                        f[e + 4] = ok ? __builtin_bit_cast(float, (uint32_t)R.v[u][1][e]) : 0.f;
                    }
                }
                *(f32x4 *)(dst + kr * VLD + c8) = f32x4{f[0], f[1], f[2], f[3]};
                *(f32x4 *)(dst + kr * VLD + c8 + 4) = f32x4{f[4], f[5], f[6], f[7]};
            }
        }
    };
    // this wave's C B^T pieces of a slab (rows t0 + r, columns kb + 4 grp ..), clamped in range
    auto load_a = [&](int k0, f32x4 (&a)[SK / 16]) {
#pragma unroll
        for (int kq = 0; kq < SK; kq += 16) {
            const int kk = min(k0 + kq + 4 * grp, Q - 4);
            a[kq / 16] = *(const f32x4 *)(arow + kk);
        }
    };

    f32x4 acc[NT];
#pragma unroll
    for (int u = 0; u < NT; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
    VRegs R0, R1;
    f32x4 a0[SK / 16], a1[SK / 16];
    auto slab = [&](int k0, VRegs &Rc, f32x4 (&ac)[SK / 16], VRegs &Rn, f32x4 (&an)[SK / 16], int buf) {
        write_v(k0, Rc, vs[buf]);
        lds_barrier();  // slab k0 complete; every wave is done with the other buffer
        load_v(k0 + SK, Rn);
        load_a(k0 + SK, an);
        if (wv) {
#pragma unroll
            for (int kq = 0; kq < SK; kq += 16) {
                const int kb = k0 + kq;
                if (kb >= k_lo && kb < k_hi) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float *vrow = vs[buf] + (kq + 4 * grp + e) * VLD + r;
#pragma unroll
                        for (int u = 0; u < NT; ++u) acc[u] = mfma_f32(ac[kq / 16][e], vrow[16 * u], acc[u]);
                    }
                }
            }
        }
    };
    load_v(g_lo, R0);
    load_a(g_lo, a0);
    // (slabs past g_hi load clamped rows, unused; no slab sits behind a branch)
    for (int k0 = g_lo; k0 < g_hi; k0 += 2 * SK) {
        slab(k0, R0, a0, R1, a1, 0);
        slab(k0 + SK, R1, a1, R0, a0, 1);
    }
    if (!wv) return;
    const float *base = which == 0 ? dCs : dBs;
    T *out = which == 0 ? dC : dB;
#pragma unroll
    for (int u = 0; u < NT; ++u) {
        const int n = u * 16 + r;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = t0 + 4 * grp + e;
            if (i < q) {
                const int64_t o = ((b * L + s + i) * G + g) * N + n;
                out[o] = from_f32<T>(acc[u][e] + base[o]);
            }
        }
    }
}

// dA[h] = sum over (b, c) of the chunk partials, likewise dD (nullable).
__global__ __launch_bounds__(256) void k_head_reduce(const float *__restrict__ part, float *dA,
                                                     float *dD, int64_t nbc, int H) {
    const int h = blockIdx.x;
    float a = 0.f, d = 0.f;
    for (int64_t k = threadIdx.x; k < nbc; k += 256) {
        a += part[(k * H + h) * 2];
        d += part[(k * H + h) * 2 + 1];
    }
    __shared__ float red[2][4];
    a = wave_sum(a);
    d = wave_sum(d);
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        red[0][wave] = a;
        red[1][wave] = d;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        dA[h] = red[0][0] + red[0][1] + red[0][2] + red[0][3];
        if (dD) dD[h] = red[1][0] + red[1][1] + red[1][2] + red[1][3];
    }
}

// ---------------------------------------------------------------------------
// Launchers.
// ---------------------------------------------------------------------------
#define SSD_BWD_DISPATCH_N(N_, ...)                                               \
    switch (N_) {                                                                 \
    case 16: { constexpr int NN = 16; __VA_ARGS__; } break;                       \
    case 32: { constexpr int NN = 32; __VA_ARGS__; } break;                       \
    case 64: { constexpr int NN = 64; __VA_ARGS__; } break;                       \
    case 128: { constexpr int NN = 128; __VA_ARGS__; } break;                     \
    case 256: { constexpr int NN = 256; __VA_ARGS__; } break;                     \
    default: return hipErrorInvalidValue;                                         \
    }
#define SSD_BWD_DISPATCH_PN(P_, N_, ...)                                          \
    do {                                                                          \
        switch (P_) {                                                             \
        case 16: { constexpr int PP = 16; SSD_BWD_DISPATCH_N(N_, __VA_ARGS__); } break; \
        case 32: { constexpr int PP = 32; SSD_BWD_DISPATCH_N(N_, __VA_ARGS__); } break; \
        case 64: { constexpr int PP = 64; SSD_BWD_DISPATCH_N(N_, __VA_ARGS__); } break; \
        case 128: { constexpr int PP = 128; SSD_BWD_DISPATCH_N(N_, __VA_ARGS__); } break; \
        default: return hipErrorInvalidValue;                                     \
        }                                                                         \
    } while (0)

hipError_t launch_state_passing_rev(const Dims &d, float *S, const float *cs, const float *dfinal,
                                    float *dinit, hipStream_t st) {
    if (d.b == 0) return hipSuccess;
    const int PN = (int)(d.P * d.N);
    dim3 grid((unsigned)((PN / 4 + 255) / 256), (unsigned)d.H, (unsigned)d.b);
    k_state_passing_rev<<<grid, 256, 0, st>>>(S, cs, dfinal, dinit, d.L, (int)d.H, PN, (int)d.Q,
                                              (int)d.nc);
    return hipGetLastError();
}

hipError_t launch_chunk_cumsum64(const Dims &d, const void *dt, const float *A, double *cs,
                                 hipStream_t st) {
    if (d.b == 0 || d.nc == 0) return hipSuccess;
    dim3 grid((unsigned)d.nc, (unsigned)d.H, (unsigned)d.b);
    if (d.dtype == 1)
        k_chunk_cumsum64<bf16><<<grid, 64, 0, st>>>((const bf16 *)dt, A, cs, d.L, (int)d.H, (int)d.Q,
                                                    (int)d.nc);
    else
        k_chunk_cumsum64<float><<<grid, 64, 0, st>>>((const float *)dt, A, cs, d.L, (int)d.H,
                                                     (int)d.Q, (int)d.nc);
    return hipGetLastError();
}

// bf16 inputs use the float32 prefix (cs), float32 inputs the float64 one (cs64).
bool chunk_bwd_frags(const Dims &d) {
    return d.dtype == 1 && d.Q <= 256 && d.Q % 16 == 0 && d.Q * d.H * d.P * 2 < (int64_t(1) << 31);
}

BwdFragBytes bwd_frag_bytes(const Dims &d) {
    const int64_t nbcg = d.b * d.nc * d.G, t16 = d.Q / 16, ncf = (d.N + 31) / 32;
    return BwdFragBytes{nbcg * t16 * ncf * 1024, nbcg * t16 * 8 * 1024, nbcg * d.Q * 4};
}

hipError_t launch_bwd_frags(const Dims &d, const void *B, const void *C, void *Gy, void *Gx,
                            void *Cf, void *Bf, float *dg, hipStream_t st) {
    if (d.b == 0 || d.nc == 0) return hipSuccess;
    dim3 grid((unsigned)(d.b * d.nc * d.G), (unsigned)(d.Q / 16));
    SSD_BWD_DISPATCH_N(d.N, {
        k_bwd_frags<NN><<<grid, 256, 0, st>>>((const bf16 *)B, (const bf16 *)C, (bf16 *)Gy,
                                              (bf16 *)Gx, (bf16 *)Cf, (bf16 *)Bf, dg, d.L, (int)d.G,
                                              (int)d.Q, (int)d.nc);
    });
    return hipGetLastError();
}

hipError_t launch_chunk_bwd(const Dims &d, const void *x, const void *dy, const void *dt,
                            const float *A, const void *B, const void *C, const void *cb,
                            const void *cbT, const void *Cf, const void *Bf, const float *dg,
                            const float *cs, const double *cs64, const float *Hs, const float *Rs,
                            const float *D, void *dx, void *ddt, float *part, hipStream_t st) {
    if (d.b == 0 || d.nc == 0) return hipSuccess;
    const unsigned grid = (unsigned)(d.b * d.nc * d.H);
    SSD_BWD_DISPATCH_PN(d.P, d.N, {
        if (chunk_bwd_frags(d))
            k_chunk_bwd_pf<PP, NN><<<grid, 256, 0, st>>>(
                (const bf16 *)x, (const bf16 *)dy, (const bf16 *)dt, A, (const bf16 *)Bf,
                (const bf16 *)Cf, (const bf16 *)cb, (const bf16 *)cbT, dg, cs, Hs, Rs, D,
                (bf16 *)dx, (bf16 *)ddt, part, d.L, (int)d.H, (int)d.G, (int)d.Q, (int)d.nc);
        else if (d.dtype == 1)
            k_chunk_bwd<bf16, PP, NN, float><<<grid, 256, 0, st>>>(
                (const bf16 *)x, (const bf16 *)dy, (const bf16 *)dt, A, (const bf16 *)B,
                (const bf16 *)C, (const bf16 *)cb, (const bf16 *)cbT, cs, Hs, Rs, D, (bf16 *)dx,
                (bf16 *)ddt, part, d.L, (int)d.H, (int)d.G, (int)d.Q, (int)d.nc);
        else
            k_chunk_bwd<float, PP, NN, double><<<grid, 256, 0, st>>>(
                (const float *)x, (const float *)dy, (const float *)dt, A, (const float *)B,
                (const float *)C, (const float *)cb, (const float *)cbT, cs64, Hs, Rs, D,
                (float *)dx, (float *)ddt, part, d.L, (int)d.H, (int)d.G, (int)d.Q, (int)d.nc);
    });
    return hipGetLastError();
}

hipError_t launch_group_bwd(const Dims &d, const void *x, const void *dy, const float *cs,
                            const double *cs64, const float *Hs, const float *Rs, float *dcb,
                            float *dcbT, float *dCs, float *dBs, hipStream_t st) {
    if (d.b == 0 || d.nc == 0) return hipSuccess;
    const unsigned grid = (unsigned)(d.b * d.nc * d.G * ((d.Q + 63) / 64));
    SSD_BWD_DISPATCH_PN(d.P, d.N, {
        // bf16 with N <= 128 and P N <= 8192: dCB and the state terms in two
        // kernels (their accumulators and prefetch fit without spills)
        constexpr bool kSplit = NN <= 128 && PP * NN <= 8192;
        if (kSplit && d.dtype == 1) {
            if constexpr (kSplit) {
                const int nbk = (int)((d.Q + 63) / 64);
                if constexpr (PP == 32 || PP == 64) {
                    const unsigned g1 = (unsigned)(d.b * d.nc * d.G * nbk);
                    k_group_dcb_rb<PP><<<g1, 64 * dcb_waves<PP>(), 0, st>>>((const bf16 *)x, (const bf16 *)dy, cs, dcb,
                                                          dcbT, d.L, (int)d.H, (int)d.G, (int)d.Q,
                                                          (int)d.nc);
                } else {
                    const unsigned g1 = (unsigned)(d.b * d.nc * d.G * (nbk * (nbk + 1) / 2));
                    k_group_dcb<PP><<<g1, 256, 0, st>>>((const bf16 *)x, (const bf16 *)dy, cs, dcb,
                                                       dcbT, d.L, (int)d.H, (int)d.G, (int)d.Q,
                                                       (int)d.nc);
                }
                if (d.Q > 64) {
                    const unsigned g2 = (unsigned)(2 * d.b * d.nc * d.G * ((d.Q + 127) / 128));
                    k_group_state<PP, NN, 8><<<g2, 512, 0, st>>>(
                        (const bf16 *)x, (const bf16 *)dy, cs, Hs, Rs, dCs, dBs, d.L, (int)d.H,
                        (int)d.G, (int)d.Q, (int)d.nc);
                } else {
                    k_group_state<PP, NN, 4><<<2 * grid, 256, 0, st>>>(
                        (const bf16 *)x, (const bf16 *)dy, cs, Hs, Rs, dCs, dBs, d.L, (int)d.H,
                        (int)d.G, (int)d.Q, (int)d.nc);
                }
            }
        } else if (d.dtype == 1)
            k_group_bwd<bf16, PP, NN, float><<<grid, 256, 0, st>>>(
                (const bf16 *)x, (const bf16 *)dy, cs, Hs, Rs, dcb, dcbT, dCs, dBs, d.L, (int)d.H,
                (int)d.G, (int)d.Q, (int)d.nc);
        else
            k_group_bwd<float, PP, NN, double><<<grid, 256, 0, st>>>(
                (const float *)x, (const float *)dy, cs64, Hs, Rs, dcb, dcbT, dCs, dBs, d.L,
                (int)d.H, (int)d.G, (int)d.Q, (int)d.nc);
    });
    return hipGetLastError();
}

hipError_t launch_group_combine(const Dims &d, const void *B, const void *C, const float *dcb,
                                const float *dcbT, const float *dCs, const float *dBs, void *dB,
                                void *dC, hipStream_t st) {
    if (d.b == 0 || d.nc == 0) return hipSuccess;
    const unsigned grid = (unsigned)(d.b * d.nc * d.G * 2 * ((d.Q + 63) / 64));
    SSD_BWD_DISPATCH_N(d.N, {
        if (d.dtype == 1)
            k_group_combine<bf16, NN><<<grid, 256, 0, st>>>((const bf16 *)B, (const bf16 *)C, dcb,
                                                           dcbT, dCs, dBs, (bf16 *)dB, (bf16 *)dC,
                                                           d.L, (int)d.G, (int)d.Q, (int)d.nc);
        else
            k_group_combine<float, NN><<<grid, 256, 0, st>>>((const float *)B, (const float *)C,
                                                            dcb, dcbT, dCs, dBs, (float *)dB,
                                                            (float *)dC, d.L, (int)d.G, (int)d.Q,
                                                            (int)d.nc);
    });
    return hipGetLastError();
}

hipError_t launch_head_reduce(const Dims &d, const float *part, float *dA, float *dD,
                              hipStream_t st) {
    k_head_reduce<<<(unsigned)d.H, 256, 0, st>>>(part, dA, dD, d.b * d.nc, (int)d.H);
    return hipGetLastError();
}

}  // namespace ssd
