// Single-pass SSD forward for bfloat16 inputs (gfx950).
//
// One workgroup per (b, c, h) does every step of the chunked algorithm for
// its chunk (Mamba-2 review, docsaid.org, section "2つのルートを半分ずつ":
// quadratic form inside the block, only the end-of-block state handed to the
// next block), so x is read from HBM once and y written once:
//
//   1. decay prefix cs of the chunk (wave scans over dt * A_h)
//   2. x^T staged in LDS twice: as is, and scaled per 32-step block by
//      v_j = exp(r_J - cs_j), r_J = cs at the block's last step
//   3. chunk state S_c^T = sum_J exp(cs_last - r_J) B_J^T x~_J (MFMA; the
//      block factors are applied Horner-style between blocks)
//   4. intra-chunk product: for output tile I, blocks J strictly before the
//      tile's own 32-block use the unmodified C B^T tile (MFMA B operand
//      straight from memory) against x~, Horner-rescaled, then one row
//      factor exp(cs_i - r); only the diagonal 32-block needs a per-element
//      mask exp(cs_i - cs_j) [j <= i]
//   5. state hand-off: wait until chunk c-1 of this (b, h) has published
//      h_{c-1}, publish h_c = exp(cs_last) h_{c-1} + S_c (2-slot ring), or
//      write final_state for the last chunk
//   6. y = intra + exp(cs_i) h_{c-1} C_i + D x_i
//
// Every factor exp(a) used in the factorised mask has a <= 0 (cs is
// non-increasing for dt >= 0, A <= 0), so nothing overflows; a factor that
// underflows multiplies a contribution that is itself below the float range.
//
// Ordering: workgroups take a ticket from an atomic counter and map it to
// (c, b, h) chunk-major, so the workgroup chunk c waits on has a smaller
// ticket, i.e. it has already started and never waits on a later one: the
// chain always drains.  The wait is also bounded (it gives up after ~0.2 s
// and the result is then wrong, never hung).  The flag is written with a
// release at agent scope after the state (L2 written back), and read with an
// acquire at agent scope (L2 invalidated) so the state is seen across XCDs.
#include "ssd_device.h"
#include "ssd_launch.h"

namespace ssd {

namespace {

constexpr int kSpinLimit = 1 << 21;

// Stage rows [0, Q) of x (row stride ld) transposed into two LDS copies:
// plain (xs) and scaled by scale[r] (xt).  Rows >= nvalid are zero.
__device__ __forceinline__ void stage_x_pair(const bf16 *__restrict__ src, int64_t ld, int rows,
                                             int cols, int nvalid, bf16 *xs, bf16 *xt, int dstride,
                                             const float *scale) {
    const int nbc = cols / 8, nbr = rows / 4;
    for (int blk = threadIdx.x; blk < nbr * nbc; blk += blockDim.x) {
        const int br = blk / nbc, bc = blk - br * nbc;
        const int r0 = br * 4, c0 = bc * 8;
        u32x4 v[4], w[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int rr = r0 + k;
            if (rr < nvalid) {
                v[k] = *(const u32x4 *)(src + (int64_t)rr * ld + c0);
                bf16x8 t = as_bf16x8(v[k]);
                const float s = scale[rr];
#pragma unroll
                for (int e = 0; e < 8; ++e) t[e] = (bf16)((float)t[e] * s);
                w[k] = as_u32x4(t);
            } else {
                v[k] = u32x4{0u, 0u, 0u, 0u};
                w[k] = v[k];
            }
        }
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            *(u32x2 *)(xs + (c0 + 2 * m) * dstride + r0) =
                u32x2{__builtin_amdgcn_perm(v[1][m], v[0][m], 0x05040100u),
                      __builtin_amdgcn_perm(v[3][m], v[2][m], 0x05040100u)};
            *(u32x2 *)(xs + (c0 + 2 * m + 1) * dstride + r0) =
                u32x2{__builtin_amdgcn_perm(v[1][m], v[0][m], 0x07060302u),
                      __builtin_amdgcn_perm(v[3][m], v[2][m], 0x07060302u)};
            *(u32x2 *)(xt + (c0 + 2 * m) * dstride + r0) =
                u32x2{__builtin_amdgcn_perm(w[1][m], w[0][m], 0x05040100u),
                      __builtin_amdgcn_perm(w[3][m], w[2][m], 0x05040100u)};
            *(u32x2 *)(xt + (c0 + 2 * m + 1) * dstride + r0) =
                u32x2{__builtin_amdgcn_perm(w[1][m], w[0][m], 0x07060302u),
                      __builtin_amdgcn_perm(w[3][m], w[2][m], 0x07060302u)};
        }
    }
}

}  // namespace

// ---------------------------------------------------------------------------
// Preparation for the single-pass kernel, one launch:
//   grid.y <  ntg : C B^T lower tiles (as k_chunk_cb), four per workgroup
//   grid.y == ntg : B^T of the chunk ([N][Q], steps contiguous, zero past
//                   the sequence end); workgroup (0, ntg) also clears the
//                   hand-off flags and the ticket counter.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_fused_prep(const bf16 *__restrict__ B,
                                                    const bf16 *__restrict__ C,
                                                    bf16 *__restrict__ cb, bf16 *__restrict__ Bt,
                                                    int *flags, int64_t nflags, int64_t L, int G,
                                                    int N, int Q, int nc) {
    const int T16 = Q / 16;
    const int ntiles = T16 * (T16 + 1) / 2;
    const int ntg = (ntiles + 3) / 4;
    const int64_t bcg = blockIdx.x;
    const int g = (int)(bcg % G);
    const int64_t bc = bcg / G;
    const int c = (int)(bc % nc);
    const int64_t b = bc / nc;
    const int64_t s = (int64_t)c * Q;
    if ((int)blockIdx.y == ntg) {
        if (bcg == 0)
            for (int64_t i = threadIdx.x; i < nflags; i += blockDim.x) flags[i] = 0;
        const int q = (int)min<int64_t>(Q, L - s);
        stage_transposed_bf16<false>(B + ((b * L + s) * G + g) * N, (int64_t)G * N, Q, N, q,
                                     Bt + bcg * (int64_t)N * Q, Q, nullptr);
        return;
    }
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int r = lane & 15, grp = lane >> 4;
    const int tile = blockIdx.y * 4 + wave;
    if (tile >= ntiles) return;
    int ti = (int)((sqrtf(8.f * tile + 1.f) - 1.f) * 0.5f);
    while ((ti + 1) * (ti + 2) / 2 <= tile) ++ti;
    while (ti * (ti + 1) / 2 > tile) --ti;
    const int tj = tile - ti * (ti + 1) / 2;
    const int64_t irow = s + ti * 16 + r, jrow = s + tj * 16 + r;
    const bool vi = irow < L, vj = jrow < L;
    const bf16 *Crow = C + ((b * L + irow) * G + g) * N;
    const bf16 *Brow = B + ((b * L + jrow) * G + g) * N;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < N; k0 += 32) {
        const int k = k0 + grp * 8;
        const u32x4 z = {0u, 0u, 0u, 0u};
        const u32x4 a = (vi && k < N) ? *(const u32x4 *)(Crow + k) : z;
        const u32x4 bb = (vj && k < N) ? *(const u32x4 *)(Brow + k) : z;
        acc = mfma_bf16(as_bf16x8(a), as_bf16x8(bb), acc);
    }
    bf16 *out = cb + bcg * (int64_t)Q * Q;
#pragma unroll
    for (int e = 0; e < 4; ++e) out[(int64_t)(ti * 16 + 4 * grp + e) * Q + tj * 16 + r] = (bf16)acc[e];
}

// ---------------------------------------------------------------------------
// The single-pass kernel.  256 threads (4 waves).  Wave w owns state n-tiles
// {w, w + 4, ...} and output tiles {w, 7 - w, 8 + w, 15 - w} (balanced over
// the triangle).
// ---------------------------------------------------------------------------
template <int P, int N>
__global__ __launch_bounds__(256) void k_ssd_fused(
    const bf16 *__restrict__ x, const bf16 *__restrict__ dt, const float *__restrict__ A,
    const bf16 *__restrict__ Bt, const bf16 *__restrict__ C, const bf16 *__restrict__ cb,
    const float *__restrict__ D, const float *init, bf16 *__restrict__ y, float *fin,
    float *ring, int *flags, int64_t L, int H, int G, int Q, int nc, int64_t nbh) {
    constexpr int PT = P / 16, NT = N / 16, NTW = (NT + 3) / 4;
    constexpr int XLD = 256 + 8, HLD = N + 8;
    static_assert(P * HLD <= P * XLD, "state staging reuses the scaled-x buffer");
    __shared__ int tk_s;
    __shared__ float cs_s[256];
    __shared__ float wsum_s[4];
    __shared__ float ref_s[8];   // r_J: cs at the last step of 32-block J
    __shared__ float vsc_s[256]; // v_j = exp(r_J(j) - cs_j)
    __shared__ bf16 xs[P * XLD];
    __shared__ bf16 xt[P * XLD];
    bf16 *hs = xt;               // reused for h_{c-1} (bf16) once x~ is consumed

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int r = lane & 15, grp = lane >> 4;
    int *ticket = flags + nbh;
    if (tid == 0) tk_s = atomicAdd(ticket, 1);
    __syncthreads();
    const int64_t t = tk_s;
    if (t >= (int64_t)nc * nbh) return;   // cannot happen when the counter was cleared
    const int c = (int)(t / nbh);
    const int64_t bh = t - (int64_t)c * nbh;
    const int64_t b = bh / H;
    const int h = (int)(bh - b * H);
    const int g = h / (H / G);
    const int64_t s = (int64_t)c * Q;
    const int q = (int)min<int64_t>(Q, L - s);
    const int nb = (q + 31) / 32;          // 32-step blocks holding data

    // 1. decay prefix
    {
        float v = (tid < q) ? (float)dt[(b * L + s + tid) * H + h] * A[h] : 0.f;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float o = __shfl_up(v, off, 64);
            if (lane >= off) v += o;
        }
        if (lane == 63) wsum_s[wave] = v;
        __syncthreads();
        for (int w = 0; w < wave; ++w) v += wsum_s[w];
        cs_s[tid] = v;  // past q: repeats the last valid value
        __syncthreads();
        if (tid < 8) ref_s[tid] = cs_s[min(32 * tid + 31, q - 1)];
        __syncthreads();
        vsc_s[tid] = __expf(ref_s[tid >> 5] - v);
        __syncthreads();
    }
    const float cs_last = cs_s[q - 1];

    // 2. stage x^T and x~^T
    const int64_t row0 = (b * L + s) * H + h;
    stage_x_pair(x + row0 * P, (int64_t)H * P, (q + 31) & ~31, P, q, xs, xt, XLD, vsc_s);
    __syncthreads();

    // 3. chunk state: acc_s[t][pt] = S^T[n = 16 (wave + 4 t) + 4 grp + e][p = 16 pt + r]
    const bf16 *Btc = Bt + ((b * nc + c) * G + g) * (int64_t)N * Q;
    f32x4 acc_s[NTW][PT];
#pragma unroll
    for (int tt = 0; tt < NTW; ++tt)
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) acc_s[tt][pt] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int J = 0; J < nb; ++J) {
        if (J > 0) {
            const float lam = __expf(ref_s[J] - ref_s[J - 1]);
#pragma unroll
            for (int tt = 0; tt < NTW; ++tt)
#pragma unroll
                for (int pt = 0; pt < PT; ++pt) acc_s[tt][pt] *= lam;
        }
        bf16x8 bx[PT];
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) bx[pt] = *(const bf16x8 *)(xt + (pt * 16 + r) * XLD + 32 * J + grp * 8);
#pragma unroll
        for (int tt = 0; tt < NTW; ++tt) {
            const int nt = wave + 4 * tt;
            if (nt < NT) {
                const bf16x8 a = as_bf16x8(*(const u32x4 *)(Btc + (int64_t)(nt * 16 + r) * Q + 32 * J + grp * 8));
#pragma unroll
                for (int pt = 0; pt < PT; ++pt) acc_s[tt][pt] = mfma_bf16(a, bx[pt], acc_s[tt][pt]);
            }
        }
    }

    // 4. intra-chunk product for this wave's output tiles
    const bf16 *cbc = cb + ((b * nc + c) * G + g) * (int64_t)Q * Q;
    const int T16 = (q + 15) / 16;
    f32x4 acc_y[4][PT];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int I = (k & 1) ? (8 * (k >> 1) + 7 - wave) : (8 * (k >> 1) + wave);
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) acc_y[k][pt] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (I >= T16) continue;
        const int il = I * 16 + r;
        const float csi = cs_s[il];
        const bf16 *grow = cbc + (int64_t)il * Q;
        const int Jd = I >> 1;
        for (int J = 0; J < Jd; ++J) {
            if (J > 0) {
                const float lam = __expf(ref_s[J] - ref_s[J - 1]);
#pragma unroll
                for (int pt = 0; pt < PT; ++pt) acc_y[k][pt] *= lam;
            }
            const bf16x8 gf = as_bf16x8(*(const u32x4 *)(grow + 32 * J + grp * 8));
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) {
                const bf16x8 ax = *(const bf16x8 *)(xt + (pt * 16 + r) * XLD + 32 * J + grp * 8);
                acc_y[k][pt] = mfma_bf16(ax, gf, acc_y[k][pt]);
            }
        }
        if (Jd > 0) {
            const float u = __expf(csi - ref_s[Jd - 1]);
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) acc_y[k][pt] *= u;
        }
        const int jl = 32 * Jd + grp * 8;
        bf16x8 bm;
        if (jl <= il) {
            const bf16x8 gv = as_bf16x8(*(const u32x4 *)(grow + jl));
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int j = jl + e;
                bm[e] = (bf16)((j <= il) ? __expf(csi - cs_s[j]) * (float)gv[e] : 0.f);
            }
        } else {
            bm = as_bf16x8(u32x4{0u, 0u, 0u, 0u});
        }
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) {
            const bf16x8 ax = *(const bf16x8 *)(xs + (pt * 16 + r) * XLD + jl);
            acc_y[k][pt] = mfma_bf16(ax, bm, acc_y[k][pt]);
        }
    }

    // 5. state hand-off
    const int64_t PN = (int64_t)P * N;
    const float *hp = nullptr;
    if (c > 0) {
        // every thread observes the flag itself, then acquires at agent scope
        int n = 0;
        while (__hip_atomic_load(flags + bh, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < c &&
               n < kSpinLimit) {
            __builtin_amdgcn_s_sleep(2);
            ++n;
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        hp = ring + (int64_t)((c - 1) & 1) * nbh * PN + bh * PN;
    } else {
        hp = init ? init + bh * PN : nullptr;
    }
    __syncthreads();  // every wave is done with x~ before hs overwrites it
    const bool have_h = hp != nullptr;
    const float lam_c = __expf(cs_last);
    float *hout = (c == nc - 1) ? (fin ? fin + bh * PN : nullptr)
                                : ring + (int64_t)(c & 1) * nbh * PN + bh * PN;
#pragma unroll
    for (int tt = 0; tt < NTW; ++tt) {
        const int nt = wave + 4 * tt;
        if (nt < NT) {
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) {
                const int p = pt * 16 + r, n0 = nt * 16 + 4 * grp;
                const f32x4 hv = have_h ? *(const f32x4 *)(hp + (int64_t)p * N + n0) : f32x4{0.f, 0.f, 0.f, 0.f};
                if (hout) *(f32x4 *)(hout + (int64_t)p * N + n0) = lam_c * hv + acc_s[tt][pt];
                bf16 hb[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) hb[e] = (bf16)hv[e];
                *(u32x2 *)(hs + p * HLD + n0) = *(const u32x2 *)hb;
            }
        }
    }
    if (c < nc - 1) {
        // each wave releases its own ring stores (L2 write-back at agent
        // scope, completion awaited) before the flag goes up
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        __syncthreads();
        if (tid == 0) __hip_atomic_store(flags + bh, c + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
        __syncthreads();
    }

    // 6. state term, skip term, store
    const bf16 *Cb = C + ((b * L + s) * G + g) * N;
    const float Dh = D ? D[h] : 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int I = (k & 1) ? (8 * (k >> 1) + 7 - wave) : (8 * (k >> 1) + wave);
        if (I >= T16) continue;
        const int il = I * 16 + r;
        const bool vi = il < q;
        if (have_h) {
            f32x4 tmp[PT];
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) tmp[pt] = f32x4{0.f, 0.f, 0.f, 0.f};
            const bf16 *crow = Cb + (int64_t)il * G * N;
#pragma unroll
            for (int k0 = 0; k0 < N; k0 += 32) {
                const int kk = k0 + grp * 8;
                const bf16x8 cf = as_bf16x8(vi ? *(const u32x4 *)(crow + kk) : u32x4{0u, 0u, 0u, 0u});
#pragma unroll
                for (int pt = 0; pt < PT; ++pt) {
                    const bf16x8 ah = *(const bf16x8 *)(hs + (pt * 16 + r) * HLD + kk);
                    tmp[pt] = mfma_bf16(ah, cf, tmp[pt]);
                }
            }
            const float ei = __expf(cs_s[il]);
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) acc_y[k][pt] += ei * tmp[pt];
        }
        if (vi) {
            const bf16 *xr = x + (row0 + (int64_t)il * H) * P;
            bf16 *yr = y + (row0 + (int64_t)il * H) * P;
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) {
                const int p0 = pt * 16 + 4 * grp;
                const u32x2 xw = *(const u32x2 *)(xr + p0);
                const bf16 *xe = (const bf16 *)&xw;
                bf16 o[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) o[e] = (bf16)(acc_y[k][pt][e] + Dh * (float)xe[e]);
                *(u32x2 *)(yr + p0) = *(const u32x2 *)o;
            }
        }
    }
}

bool fused_supported(const Dims &d) {
    return d.dtype == 1 && d.P == 64 && d.N == 128 && d.Q <= 256 && d.nc >= 1;
}

hipError_t launch_fused_prep(const Dims &d, const void *B, const void *C, void *cb, void *Bt,
                             int *flags, hipStream_t st) {
    const int T16 = (int)(d.Q / 16);
    const int ntg = (T16 * (T16 + 1) / 2 + 3) / 4;
    dim3 grid((unsigned)(d.b * d.nc * d.G), (unsigned)(ntg + 1));
    k_fused_prep<<<grid, 256, 0, st>>>((const bf16 *)B, (const bf16 *)C, (bf16 *)cb, (bf16 *)Bt, flags,
                                       d.b * d.H + 1, d.L, (int)d.G, (int)d.N, (int)d.Q, (int)d.nc);
    return hipGetLastError();
}

hipError_t launch_fused_main(const Dims &d, const void *x, const void *dt, const float *A,
                             const void *Bt, const void *C, const void *cb, const float *D,
                             const float *init, void *y, float *fin, float *ring, int *flags,
                             hipStream_t st) {
    const unsigned grid = (unsigned)(d.b * d.nc * d.H);
    k_ssd_fused<64, 128><<<grid, 256, 0, st>>>(
        (const bf16 *)x, (const bf16 *)dt, A, (const bf16 *)Bt, (const bf16 *)C, (const bf16 *)cb, D,
        init, (bf16 *)y, fin, ring, flags, d.L, (int)d.H, (int)d.G, (int)d.Q, (int)d.nc, d.b * d.H);
    return hipGetLastError();
}

}  // namespace ssd
