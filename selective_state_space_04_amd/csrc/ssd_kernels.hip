// SSD layer kernels for gfx950 (MI355X): the steps of the chunked algorithm
// and the single-token decode step.
//
// Notation (per batch row b, head h, group g = h / (H / G), chunk c covering
// steps s = c Q .. s + q - 1 with q = min(Q, L - s)):
//   cs_i      = sum_{k <= i} dt_{s+k} A_h            (decay prefix, log domain)
//   G_ij      = C_{s+i} . B_{s+j}                      (shared by a group's heads)
//   S_c       = sum_j exp(cs_{q-1} - cs_j) x_{s+j} B_{s+j}^T        [P, N]
//   hprev_c   = state entering chunk c
//   y_{s+i}   = sum_{j <= i} exp(cs_i - cs_j) G_ij x_{s+j}
//               + exp(cs_i) hprev_c C_{s+i} + D_h x_{s+i}
// (Mamba-2 review, docsaid.org: section "A を一つの数に簡略化する" for
// M = L o (C B^T) with L_ij the product of decays; section "2つのルートを半分ずつ"
// for the block split into a quadratic part inside blocks and states across
// them.)  The within-chunk weights exp(cs_{q-1} - cs_j) on the chunk state are
// what makes the split exact.
#include <algorithm>

#include "ssd_device.h"
#include "ssd_launch.h"

namespace ssd {

// ---------------------------------------------------------------------------
// Decay prefix: one wave per (b, h, c).  Each lane sums up to 4 consecutive
// steps serially, then a log-depth inclusive scan across the 64 lanes joins
// them.  Entries past a short chunk's end repeat its last value (dt treated
// as 0 there), so every consumer sees finite numbers.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(64) void k_chunk_cumsum(const T *__restrict__ dt,
                                                     const float *__restrict__ A,
                                                     float *__restrict__ cs, int64_t L, int H,
                                                     int Q, int nc) {
    const int c = blockIdx.x, h = blockIdx.y;
    const int64_t b = blockIdx.z;
    const int lane = threadIdx.x;
    const int64_t s = (int64_t)c * Q;
    const int q = (int)min<int64_t>(Q, L - s);
    const float Ah = A[h];
    const int per = (Q + 63) / 64;  // <= 4
    float v[4];
    float run = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int i = lane * per + e;
        float d = 0.f;
        if (e < per && i < q) d = to_f32(dt[((b * L) + s + i) * H + h]) * Ah;
        run += d;
        v[e] = run;
    }
    float tot = run;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const float o = __shfl_up(tot, off, 64);
        if (lane >= off) tot += o;
    }
    const float excl = tot - run;
    float *out = cs + (((int64_t)b * H + h) * nc + c) * Q;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int i = lane * per + e;
        if (e < per && i < Q) out[i] = v[e] + excl;
    }
}

// The same prefix over the preprocessed step dt_eff = dt_effective(dt) (bias,
// softplus, clamp), and, when sc is given, the input scale of every step
// (zero past a short chunk's end, where x is zero too).
template <typename T>
__global__ __launch_bounds__(64) void k_chunk_cumsum_opts(const T *__restrict__ dt,
                                                          const float *__restrict__ A, DtOpts o,
                                                          float *__restrict__ cs,
                                                          float *__restrict__ sc, int64_t L,
                                                          int H, int Q, int nc) {
    const int c = blockIdx.x, h = blockIdx.y;
    const int64_t b = blockIdx.z;
    const int lane = threadIdx.x;
    const int64_t s = (int64_t)c * Q;
    const int q = (int)min<int64_t>(Q, L - s);
    const float Ah = A[h];
    const int per = (Q + 63) / 64;
    float v[4], sv[4];
    float run = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int i = lane * per + e;
        float d = 0.f, sx = 0.f;
        if (e < per && i < q) {
            const float de = dt_effective(to_f32(dt[((b * L) + s + i) * H + h]), h, o);
            d = de * Ah;
            sx = input_scale(de, Ah, o.scale);
        }
        run += d;
        v[e] = run;
        sv[e] = sx;
    }
    float tot = run;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const float t = __shfl_up(tot, off, 64);
        if (lane >= off) tot += t;
    }
    const float excl = tot - run;
    const int64_t base = (((int64_t)b * H + h) * nc + c) * Q;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int i = lane * per + e;
        if (e < per && i < Q) {
            cs[base + i] = v[e] + excl;
            if (sc) sc[base + i] = sv[e];
        }
    }
}

// ---------------------------------------------------------------------------
// C B^T per (b, c, g): one wave per 16 x 16 tile on or below the diagonal,
// K = N in MFMA steps.  A operand = C rows (m = i), B operand = B rows
// (n = j); both are read straight from global memory with the contraction
// index contiguous.  When cbT is given, the same tiles are also written
// transposed (cbT[j][i] = C_i . B_j), which the gradient kernels read with
// the step index i contiguous.
// ---------------------------------------------------------------------------
template <typename T, int N>
__global__ __launch_bounds__(256) void k_chunk_cb(const T *__restrict__ B, const T *__restrict__ C,
                                                  T *__restrict__ cb, T *__restrict__ cbT,
                                                  int64_t L, int G, int Q, int nc) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int r = lane & 15, grp = lane >> 4;
    const int T16 = Q / 16;
    const int ntiles = T16 * (T16 + 1) / 2;
    const int tile = blockIdx.y * 4 + wave;
    if (tile >= ntiles) return;
    int ti = (int)((sqrtf(8.f * tile + 1.f) - 1.f) * 0.5f);
    while ((ti + 1) * (ti + 2) / 2 <= tile) ++ti;
    while (ti * (ti + 1) / 2 > tile) --ti;
    const int tj = tile - ti * (ti + 1) / 2;
    const int64_t bcg = blockIdx.x;
    const int g = (int)(bcg % G);
    const int64_t bc = bcg / G;
    const int c = (int)(bc % nc);
    const int64_t b = bc / nc;
    const int64_t s = (int64_t)c * Q;
    const int64_t irow = s + ti * 16 + r, jrow = s + tj * 16 + r;
    const bool vi = irow < L, vj = jrow < L;
    // rows past L read row s (always present) and are zeroed after the load:
    // all of a lane's loads issue before its first MFMA, with no branch
    const T *Crow = C + ((b * L + (vi ? irow : s)) * G + g) * N;
    const T *Brow = B + ((b * L + (vj ? jrow : s)) * G + g) * N;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if constexpr (sizeof(T) == 2) {
        constexpr int NI = (N + 31) / 32;
        const u32x4 z = {0u, 0u, 0u, 0u};
        u32x4 a[NI], bb[NI];
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int k = i * 32 + grp * 8;
            a[i] = *(const u32x4 *)(Crow + min(k, N - 8));
            bb[i] = *(const u32x4 *)(Brow + min(k, N - 8));
            if (!vi || k >= N) a[i] = z;
            if (!vj || k >= N) bb[i] = z;
        }
#pragma unroll
        for (int i = 0; i < NI; ++i) acc = mfma_bf16(as_bf16x8(a[i]), as_bf16x8(bb[i]), acc);
    } else {
        constexpr int NI = N / 16;
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        f32x4 a[NI], bb[NI];
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int k = i * 16 + grp * 4;
            a[i] = *(const f32x4 *)(Crow + k);
            bb[i] = *(const f32x4 *)(Brow + k);
            if (!vi) a[i] = z;
            if (!vj) bb[i] = z;
        }
#pragma unroll
        for (int i = 0; i < NI; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc = mfma_f32(a[i][e], bb[i][e], acc);
    }
    const int64_t off = (((int64_t)b * nc + c) * G + g) * (int64_t)Q * Q;
    T *out = cb + off;
#pragma unroll
    for (int e = 0; e < 4; ++e)
        out[(int64_t)(ti * 16 + 4 * grp + e) * Q + tj * 16 + r] = from_f32<T>(acc[e]);
    if (cbT) {
        T v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = from_f32<T>(acc[e]);
        T *dst = cbT + off + (int64_t)(tj * 16 + r) * Q + ti * 16 + 4 * grp;
        if constexpr (sizeof(T) == 2) *(u32x2 *)dst = *(const u32x2 *)v;
        else *(f32x4 *)dst = *(const f32x4 *)v;
    }
}

// ---------------------------------------------------------------------------
// Chunk state S_c^T[n][p] = sum_j B_j[n] (w_j x_j[p]), one workgroup per
// (b, c, h).  w_j = exp(cs_{q-1} - cs_j) (decay to the chunk end) for the
// forward state; with FROM_START, w_j = exp(cs_j) (decay from the chunk
// start), which with (x, B) -> (dy, C) gives the gradient that a chunk's
// outputs send back to the state entering it.  bf16: 64-step slabs of x (pre-scaled by w_j) and B are staged
// in LDS transposed (step index contiguous) so each MFMA fragment is one
// 16-byte LDS read (float32 inputs: k_chunk_state_f32).  Wave w owns
// n-tiles w, w + 4, ...
// ---------------------------------------------------------------------------
// One thread's share of a [64 x COLS] bf16 slab in registers: blocks of 4
// rows x 8 columns, block tid + 256 i, as four 16-byte row pieces; rows at
// or past nvalid read as zero.
template <int COLS>
struct SlabRegs {
    static constexpr int NBLK = 16 * (COLS / 8);
    static constexpr int PER = (NBLK + 255) / 256;
    u32x4 v[PER][4];
};

template <int COLS>
__device__ __forceinline__ void slab_load(SlabRegs<COLS> &st, const bf16 *__restrict__ src, int64_t ld,
                                          int nvalid) {
    constexpr int NBC = COLS / 8;
#pragma unroll
    for (int i = 0; i < SlabRegs<COLS>::PER; ++i) {
        const int blk = threadIdx.x + 256 * i;
        if (blk < SlabRegs<COLS>::NBLK) {
            const int r0 = (blk / NBC) * 4, c0 = (blk % NBC) * 8;
#pragma unroll
            for (int k = 0; k < 4; ++k)
                st.v[i][k] = r0 + k < nvalid ? *(const u32x4 *)(src + (int64_t)(r0 + k) * ld + c0)
                                             : u32x4{0u, 0u, 0u, 0u};
        }
    }
}

// Write the slab transposed: dst[c * dstride + r] = slab[r][c] (times
// scale[r] when SCALE, rounded back to bf16), as in stage_transposed_bf16.
template <bool SCALE, int COLS>
__device__ __forceinline__ void slab_write_transposed(const SlabRegs<COLS> &st, bf16 *dst, int dstride,
                                                      const float *scale) {
    constexpr int NBC = COLS / 8;
#pragma unroll
    for (int i = 0; i < SlabRegs<COLS>::PER; ++i) {
        const int blk = threadIdx.x + 256 * i;
        if (blk < SlabRegs<COLS>::NBLK) {
            const int r0 = (blk / NBC) * 4, c0 = (blk % NBC) * 8;
            u32x4 v[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                v[k] = st.v[i][k];
                if constexpr (SCALE) {
                    bf16x8 t = as_bf16x8(v[k]);
                    const float w = scale[r0 + k];
#pragma unroll
                    for (int e = 0; e < 8; ++e) t[e] = (bf16)((float)t[e] * w);
                    v[k] = as_u32x4(t);
                }
            }
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const uint32_t lo01 = __builtin_amdgcn_perm(v[1][m], v[0][m], 0x05040100u);
                const uint32_t lo23 = __builtin_amdgcn_perm(v[3][m], v[2][m], 0x05040100u);
                const uint32_t hi01 = __builtin_amdgcn_perm(v[1][m], v[0][m], 0x07060302u);
                const uint32_t hi23 = __builtin_amdgcn_perm(v[3][m], v[2][m], 0x07060302u);
                *(u32x2 *)(dst + (c0 + 2 * m) * dstride + r0) = u32x2{lo01, lo23};
                *(u32x2 *)(dst + (c0 + 2 * m + 1) * dstride + r0) = u32x2{hi01, hi23};
            }
        }
    }
}

template <typename T, int P, int N, bool FROM_START>
__global__ __launch_bounds__(256) void k_chunk_state(const T *__restrict__ x,
                                                     const T *__restrict__ B,
                                                     const float *__restrict__ cs,
                                                     float *__restrict__ S, int64_t L, int H,
                                                     int G, int Q, int nc,
                                                     const float *__restrict__ sc) {
    constexpr int PT = P / 16, NT = N / 16, NTW = (NT + 3) / 4;
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

    __shared__ float w_s[256];
    const float *csc = cs + (((int64_t)b * H + h) * nc + c) * Q;
    const float cs_last = csc[q - 1];
    const float *scc = sc ? sc + (((int64_t)b * H + h) * nc + c) * Q : nullptr;
    for (int j = threadIdx.x; j < Q; j += 256)
        w_s[j] = (FROM_START ? __expf(csc[j]) : __expf(cs_last - csc[j])) * (scc ? scc[j] : 1.f);
    __syncthreads();

    f32x4 acc[NTW][PT];
#pragma unroll
    for (int t = 0; t < NTW; ++t)
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) acc[t][pt] = f32x4{0.f, 0.f, 0.f, 0.f};

    const T *xb = x + ((b * L + s) * H + h) * P;
    const T *Bb = B + ((b * L + s) * G + g) * N;
    static_assert(sizeof(T) == 2, "float32 inputs use k_chunk_state_f32");
    {
        constexpr int SL = 64, LD = SL + 8;
        __shared__ bf16 xs[P * LD];
        __shared__ bf16 bs[N * LD];
        // slab jb + SL is loaded into registers while slab jb is multiplied;
        // the barriers only order LDS, so the loads stay in flight
        SlabRegs<P> rx;
        SlabRegs<N> rb;
        slab_load(rx, xb, (int64_t)H * P, min(SL, q));
        slab_load(rb, Bb, (int64_t)G * N, min(SL, q));
        for (int jb = 0; jb < q; jb += SL) {
            slab_write_transposed<true>(rx, xs, LD, w_s + jb);
            slab_write_transposed<false>(rb, bs, LD, nullptr);
            lds_barrier();
            if (jb + SL < q) {
                const int nv = min(SL, q - jb - SL);
                slab_load(rx, xb + (int64_t)(jb + SL) * H * P, (int64_t)H * P, nv);
                slab_load(rb, Bb + (int64_t)(jb + SL) * G * N, (int64_t)G * N, nv);
            }
#pragma unroll
            for (int kk = 0; kk < SL; kk += 32) {
                bf16x8 bx[PT];
#pragma unroll
                for (int pt = 0; pt < PT; ++pt)
                    bx[pt] = *(const bf16x8 *)(xs + (pt * 16 + r) * LD + kk + grp * 8);
#pragma unroll
                for (int t = 0; t < NTW; ++t) {
                    const int nt = wave + 4 * t;
                    if (nt < NT) {
                        const bf16x8 ab = *(const bf16x8 *)(bs + (nt * 16 + r) * LD + kk + grp * 8);
#pragma unroll
                        for (int pt = 0; pt < PT; ++pt) acc[t][pt] = mfma_bf16(ab, bx[pt], acc[t][pt]);
                    }
                }
            }
            lds_barrier();
        }
    }
    // acc[t][pt][e] = S^T[n = nt*16 + 4 grp + e][p = pt*16 + r]
    float *So = S + (((b * nc + c) * H + h) * (int64_t)P) * N;
#pragma unroll
    for (int t = 0; t < NTW; ++t) {
        const int nt = wave + 4 * t;
        if (nt < NT) {
#pragma unroll
            for (int pt = 0; pt < PT; ++pt)
                *(f32x4 *)(So + (int64_t)(pt * 16 + r) * N + nt * 16 + 4 * grp) = acc[t][pt];
        }
    }
}

// s_waitcnt vmcnt(n) lgkmcnt(0) for a run-time n (the instruction takes an
// immediate); n past 47 waits for everything.
__device__ __forceinline__ void wait_vmcnt_lgkm0(int n) {
    switch (n) {
    case 0: __builtin_amdgcn_s_waitcnt(112); break;
    case 1: __builtin_amdgcn_s_waitcnt(113); break;
    case 2: __builtin_amdgcn_s_waitcnt(114); break;
    case 3: __builtin_amdgcn_s_waitcnt(115); break;
    case 4: __builtin_amdgcn_s_waitcnt(116); break;
    case 5: __builtin_amdgcn_s_waitcnt(117); break;
    case 6: __builtin_amdgcn_s_waitcnt(118); break;
    case 7: __builtin_amdgcn_s_waitcnt(119); break;
    case 8: __builtin_amdgcn_s_waitcnt(120); break;
    case 9: __builtin_amdgcn_s_waitcnt(121); break;
    case 10: __builtin_amdgcn_s_waitcnt(122); break;
    case 11: __builtin_amdgcn_s_waitcnt(123); break;
    case 12: __builtin_amdgcn_s_waitcnt(124); break;
    case 13: __builtin_amdgcn_s_waitcnt(125); break;
    case 14: __builtin_amdgcn_s_waitcnt(126); break;
    case 15: __builtin_amdgcn_s_waitcnt(127); break;
    case 16: __builtin_amdgcn_s_waitcnt(16496); break;
    case 17: __builtin_amdgcn_s_waitcnt(16497); break;
    case 18: __builtin_amdgcn_s_waitcnt(16498); break;
    case 19: __builtin_amdgcn_s_waitcnt(16499); break;
    case 20: __builtin_amdgcn_s_waitcnt(16500); break;
    case 21: __builtin_amdgcn_s_waitcnt(16501); break;
    case 22: __builtin_amdgcn_s_waitcnt(16502); break;
    case 23: __builtin_amdgcn_s_waitcnt(16503); break;
    case 24: __builtin_amdgcn_s_waitcnt(16504); break;
    case 25: __builtin_amdgcn_s_waitcnt(16505); break;
    case 26: __builtin_amdgcn_s_waitcnt(16506); break;
    case 27: __builtin_amdgcn_s_waitcnt(16507); break;
    case 28: __builtin_amdgcn_s_waitcnt(16508); break;
    case 29: __builtin_amdgcn_s_waitcnt(16509); break;
    case 30: __builtin_amdgcn_s_waitcnt(16510); break;
    case 31: __builtin_amdgcn_s_waitcnt(16511); break;
    case 32: __builtin_amdgcn_s_waitcnt(32880); break;
    case 33: __builtin_amdgcn_s_waitcnt(32881); break;
    case 34: __builtin_amdgcn_s_waitcnt(32882); break;
    case 35: __builtin_amdgcn_s_waitcnt(32883); break;
    case 36: __builtin_amdgcn_s_waitcnt(32884); break;
    case 37: __builtin_amdgcn_s_waitcnt(32885); break;
    case 38: __builtin_amdgcn_s_waitcnt(32886); break;
    case 39: __builtin_amdgcn_s_waitcnt(32887); break;
    case 40: __builtin_amdgcn_s_waitcnt(32888); break;
    case 41: __builtin_amdgcn_s_waitcnt(32889); break;
    case 42: __builtin_amdgcn_s_waitcnt(32890); break;
    case 43: __builtin_amdgcn_s_waitcnt(32891); break;
    case 44: __builtin_amdgcn_s_waitcnt(32892); break;
    case 45: __builtin_amdgcn_s_waitcnt(32893); break;
    case 46: __builtin_amdgcn_s_waitcnt(32894); break;
    case 47: __builtin_amdgcn_s_waitcnt(32895); break;
    default: __builtin_amdgcn_s_waitcnt(0x0070); break;
    }
}

// ---------------------------------------------------------------------------
// Chunk states for bfloat16 with P in {32, 64}, N in {64, 128} and Q a
// multiple of 32 (both backward passes and the staged forward use it): one
// workgroup per (b, c, g, part of the group's heads), one wave per 16-column
// tile of N.  The chunk's B rows are read once into registers (as MFMA
// fragments, through LDS) and x streams in head by head: each head's rows
// are loaded into registers two heads ahead and stored to one of two LDS
// buffers (row-major, pair-swizzled) one head ahead.  The MFMA operands,
// which contract over the steps, are read with transposing LDS reads
// (ds_read_b64_tr_b16), two per fragment.  The step weights w_j
// (exp(cs_e - cs_j), or exp(cs_j) from the chunk start, times the optional
// input factor) scale the B^T fragments.  Per head: one barrier, the loads of
// head + 2 and the next prefix, multiply, store S, the next head's weights
// and rows to LDS.  No load sits behind a branch (heads past the part's end
// repeat its last head; copy indices are clamped), so the compiler's
// counted waits leave the later heads' loads in flight.  (Direct global-to-
// LDS copies would save the registers, but after one the compiler makes
// every LDS read wait for all copies in flight.)
// ---------------------------------------------------------------------------
template <int P, int N, bool FROM_START>
__global__ __launch_bounds__(64 * (N / 16)) void k_chunk_state_mh(const bf16 *__restrict__ x,
                                                        const bf16 *__restrict__ B,
                                                        const float *__restrict__ cs,
                                                        float *__restrict__ S, int64_t L, int H,
                                                        int G, int Q, int nc,
                                                        const float *__restrict__ sc, int nparts) {
    constexpr int XROWB = P * 2, BROWB = N * 2;
    constexpr int PT = P / 16, NT = N / 16, NW = NT;  // one wave per 16-column tile of N
    constexpr int XSLOT = 256 * XROWB;
    constexpr int XCPR = XROWB / 16, XRPC = 1024 / XROWB;   // x: 16-byte chunks per row, rows per KiB
    constexpr int CPW = (256 * XROWB / 1024 + NW - 1) / NW; // KiB pieces of a head per wave
    static_assert(NT % 4 == 0 && (P == 32 || P == 64), "shape");
    constexpr int LDSB = 2 * XSLOT > 256 * BROWB ? 2 * XSLOT : 256 * BROWB;  // B is staged here first
    __shared__ __attribute__((aligned(16))) unsigned char xsm[LDSB];
    __shared__ float wsm[2][256];
    const int64_t wg = xcd_remap(blockIdx.x, gridDim.x);
    const int part = (int)(wg % nparts);
    const int64_t bcg = wg / nparts;
    const int g = (int)(bcg % G);
    const int64_t bc = bcg / G;
    const int c = (int)(bc % nc);
    const int64_t b = bc / nc;
    const int64_t s = (int64_t)c * Q;
    const int q = (int)min<int64_t>(Q, L - s);
    const int hpg = H / G, hpp = (hpg + nparts - 1) / nparts;
    const int h_lo = g * hpg + part * hpp, h_hi = min(h_lo + hpp, (g + 1) * hpg);
    const int nh = h_hi - h_lo;
    if (nh <= 0) return;  // uniform over the workgroup; no barrier reached
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int grp = lane >> 4;
    const int nk = Q / 32;

    // B rows of the chunk through LDS, into registers as this wave's fragments
    // (rows k0 + 8 grp .. of column tile `wave`)
    copy_tile_to_lds<BROWB, NW>(B + ((b * L + s) * G + g) * N, (int64_t)G * N, Q, q, xsm, wave, lane);
    __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
    __syncthreads();
    bf16x8 bfr[8];
#pragma unroll
    for (int k = 0; k < 8; ++k)
        bfr[k] = k < nk ? frag_tr<BROWB>(xsm, 32 * k, wave * 16, lane) : bf16x8{};
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the reads are done before the buffers are reused
    __syncthreads();

    // x of one head: this wave's KiB pieces k = wave, wave + NW, ... (lane's
    // 16 bytes: row k XRPC + lane / XCPR, source chunk swizzled like
    // copy_tile_to_lds), clamped so every wave issues CPW loads
    const int ncopy = Q * XROWB / 1024;
    struct XRegs {
        u32x4 v[CPW];
    };
    auto load_x = [&](int hh, XRegs &R) {
        const bf16 *src = x + ((b * L + s) * H + h_lo + min(hh, nh - 1)) * P;
#pragma unroll
        for (int i = 0; i < CPW; ++i) {
            const int k = min(wave + NW * i, ncopy - 1);
            const int row = k * XRPC + lane / XCPR;
            const int chunk = tr_chunk_slot<XROWB>(row, lane % XCPR);
            R.v[i] = *(const u32x4 *)(src + (int64_t)min(row, q - 1) * H * P + chunk * 8);
        }
    };
    auto write_x = [&](const XRegs &R, int buf) {
#pragma unroll
        for (int i = 0; i < CPW; ++i) {
            const int k = wave + NW * i;
            if (k < ncopy) *(u32x4 *)(xsm + buf * XSLOT + k * 1024 + lane * 16) = R.v[i];
        }
    };
    // thread tid < 256 holds step j = tid of a head: its weight (zero past q);
    // every thread loads (the rest a clamped duplicate), so the counts are uniform
    float n_csj = 0.f, n_cse = 0.f, n_scj = 1.f;
    // this batch row's input factors [H][nc][Q] (empty without them)
    const auto rs_sc = buf_rsrc(sc ? sc + (int64_t)b * H * nc * Q : nullptr, sc ? (uint32_t)(H * nc * Q * 4) : 0u);
    auto load_cs = [&](int hh) {
        const int h = h_lo + min(hh, nh - 1);
        const int64_t o = (((int64_t)b * H + h) * nc + c) * Q;
        const int j = min(tid & 255, q - 1);
        n_csj = cs[o + j];
        n_cse = cs[o + q - 1];
        // (no input factor: the resource is empty and the load reads zero)
        n_scj = buf_ldf(rs_sc, (uint32_t)((o - (int64_t)b * H * nc * Q) + j) * 4u) + (sc ? 0.f : 1.f);
    };
    auto weight = [&]() {
        return tid < q ? (FROM_START ? __expf(n_csj) : __expf(n_cse - n_csj)) * n_scj : 0.f;
    };

    XRegs X0, X1;
    load_cs(0);
    load_x(0, X0);
    load_x(1, X1);
    if (tid < 256) wsm[0][tid] = weight();
    write_x(X0, 0);
    load_x(2, X0);
    load_cs(1);
    // Head hh: its rows and weights sit in LDS buffer hh & 1; the rows of
    // head hh + 1 are in registers (X1 for even hh), those of hh + 2 loading.
    auto head = [&](int hh, XRegs &Xnext, XRegs &Xfree) {
        lds_barrier();  // buffer hh & 1 complete; every wave is done with buffer (hh + 1) & 1
        const int bi = hh & 1;
        f32x4 acc[PT];
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) acc[pt] = f32x4{0.f, 0.f, 0.f, 0.f};
        const float *w = wsm[bi];
        const unsigned char *xt = xsm + bi * XSLOT;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            if (k < nk) {
                bf16x8 bx[PT];
#pragma unroll
                for (int pt = 0; pt < PT; ++pt) bx[pt] = frag_tr<XROWB>(xt, 32 * k, pt * 16, lane);
                const f32x4 w0 = *(const f32x4 *)(w + 32 * k + 8 * grp);
                const f32x4 w1 = *(const f32x4 *)(w + 32 * k + 8 * grp + 4);
                bf16x8 ab = bfr[k];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    ab[e] = (bf16)((float)ab[e] * w0[e]);
                    ab[e + 4] = (bf16)((float)ab[e + 4] * w1[e]);
                }
#pragma unroll
                for (int pt = 0; pt < PT; ++pt) acc[pt] = mfma_bf16(ab, bx[pt], acc[pt]);
            }
        }
        // acc[pt][e] = S^T[n = 16 wave + 4 grp + e][p = 16 pt + r]
        float *So = S + (((b * nc + c) * H + h_lo + min(hh, nh - 1)) * (int64_t)P) * N;
        const int r = lane & 15;
#pragma unroll
        for (int pt = 0; pt < PT; ++pt)
            *(f32x4 *)(So + (int64_t)(pt * 16 + r) * N + wave * 16 + 4 * grp) = acc[pt];
        // head hh + 1 into the other buffer, then the loads of head hh + 3
        if (tid < 256) wsm[bi ^ 1][tid] = weight();
        write_x(Xnext, bi ^ 1);
        load_x(hh + 3, Xnext);
        load_cs(hh + 2);
        (void)Xfree;
    };
    // (no branch around a head: an odd count repeats the last head, whose
    // second result equals the first)
    for (int hh = 0; hh < nh; hh += 2) {
        head(hh, X1, X0);
        head(hh + 1, X0, X1);
    }
}

// ---------------------------------------------------------------------------
// Inter-chunk recurrence, in place: S[c] -> hprev[c].  Each thread owns four
// consecutive state elements of one (b, h) and walks the chunks in order.
// The chunk states do not depend on the running state, so they load in
// batches of U, one batch ahead of the one being combined (two batches in
// flight).  The loads are unconditional (a batch past the end repeats the
// last chunk) and so are the full batches' stores; only the last partial
// batch branches.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_state_passing(float *__restrict__ S,
                                                       const float *__restrict__ cs,
                                                       const float *init, float *fin, int64_t L,
                                                       int H, int PN, int Q, int nc) {
    const int h = blockIdx.y;
    const int64_t b = blockIdx.z;
    const int e0 = (blockIdx.x * 256 + threadIdx.x) * 4;
    if (e0 >= PN) return;
    const int64_t bh = b * H + h;
    f32x4 hv = init ? *(const f32x4 *)(init + bh * PN + e0) : f32x4{0.f, 0.f, 0.f, 0.f};
    const float *csb = cs + bh * (int64_t)nc * Q;
    auto at = [&](int c) { return S + (((b * nc + c) * H + h) * (int64_t)PN) + e0; };
    constexpr int U = 8;
    f32x4 sa[U], sb[U];
    float la[U], lb[U];
    auto load = [&](int c0, f32x4(&v)[U], float(&l)[U]) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = min(c0 + u, nc - 1);
            const int last = (int)min<int64_t>(Q, L - (int64_t)c * Q) - 1;
            l[u] = __expf(csb[(int64_t)c * Q + last]);
            v[u] = *(const f32x4 *)at(c);
        }
    };
    auto step = [&](int c0, const f32x4(&v)[U], const float(&l)[U]) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            *(f32x4 *)at(c0 + u) = hv;
            hv = l[u] * hv + v[u];
        }
    };
    auto tail = [&](int c0, const f32x4(&v)[U], const float(&l)[U]) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (c0 + u < nc) {
                *(f32x4 *)at(c0 + u) = hv;
                hv = l[u] * hv + v[u];
            }
        }
    };
    // two register batches used in turn (a copy from one to the other would
    // wait for the batch in flight)
    load(0, sa, la);
    for (int c0 = 0;;) {
        if (c0 + U > nc) {
            tail(c0, sa, la);
            break;
        }
        load(c0 + U, sb, lb);
        step(c0, sa, la);
        c0 += U;
        if (c0 + U > nc) {
            tail(c0, sb, lb);
            break;
        }
        load(c0 + U, sa, la);
        step(c0, sb, lb);
        c0 += U;
    }
    if (fin) *(f32x4 *)(fin + bh * PN + e0) = hv;
}

// final_state for an empty sequence: a copy of init (or zeros).
__global__ __launch_bounds__(256) void k_copy_state(const float *init, float *fin, int64_t n) {
    const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i >= n) return;
    const f32x4 v = init ? *(const f32x4 *)(init + i) : f32x4{0.f, 0.f, 0.f, 0.f};
    *(f32x4 *)(fin + i) = v;
}

// ---------------------------------------------------------------------------
// Intra-chunk masked product + output combine, one workgroup per (b, c, h).
// Computed transposed, Y^T[p][i], so each lane ends up owning one output row
// i and four consecutive channels p (one 8- or 16-byte store):
//   off term:  Y^T += h[p][n] C[i][n]      (A = state rows, B = C rows)
//   scale:     Y^T[:, i] *= exp(cs_i)
//   intra:     Y^T += x^T[p][j] M^T[j][i], M^T[j][i] = exp(cs_i - cs_j) G[i][j] (j <= i)
//   skip:      Y^T[p][i] += D_h x[i][p]
// The 16-wide output tiles are dealt to the four waves in a snake order so
// the triangular work is balanced.  bf16: x^T and the state (as bf16) are
// staged in LDS.  float32 inputs run k_chunk_scan_f32; this kernel's f32
// branch, with operands read from global memory, serves only chunks whose y
// rows span 2^31 bytes or more (beyond one buffer resource).
// ---------------------------------------------------------------------------
template <typename T, int P, int N>
__global__ __launch_bounds__(256) void k_chunk_scan(const T *__restrict__ x, const T *__restrict__ C,
                                                    const T *__restrict__ cb,
                                                    const float *__restrict__ cs,
                                                    const float *__restrict__ hprev,
                                                    const float *__restrict__ D, T *__restrict__ y,
                                                    int64_t L, int H, int G, int Q, int nc,
                                                    const float *__restrict__ sc) {
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

    __shared__ float cs_s[256], sc_s[256];
    const float *csc = cs + (((int64_t)b * H + h) * nc + c) * Q;
    const float *scc = sc ? sc + (((int64_t)b * H + h) * nc + c) * Q : nullptr;
    for (int j = threadIdx.x; j < Qp; j += 256) {
        cs_s[j] = csc[min(j, Q - 1)];
        sc_s[j] = scc ? scc[min(j, Q - 1)] : 1.f;
    }

    const T *cbc = cb + (((int64_t)b * nc + c) * G + g) * (int64_t)Q * Q;
    const float *hp = hprev ? hprev + (((b * nc + c) * H + h) * (int64_t)P) * N : nullptr;
    const float Dh = D ? D[h] : 0.f;
    const int64_t row0 = (b * L + s) * H + h;  // (row of step s, head h) in x / y
    const T *Cb = C + ((b * L + s) * G + g) * N;

    constexpr int XLD = 256 + 8, HLD = N + 8;
    __shared__ bf16 xs[sizeof(T) == 2 ? P * XLD : 1];
    __shared__ bf16 hs[sizeof(T) == 2 ? P * HLD : 1];
    if constexpr (sizeof(T) == 2) {
        stage_transposed_bf16<false>((const bf16 *)x + row0 * P, (int64_t)H * P, Qp, P, q, xs, XLD,
                                     nullptr);
        if (hp) {
            for (int idx = threadIdx.x; idx < P * N / 8; idx += 256) {
                const int p = idx / (N / 8), n0 = (idx - p * (N / 8)) * 8;
                const f32x4 a0 = *(const f32x4 *)(hp + (int64_t)p * N + n0);
                const f32x4 a1 = *(const f32x4 *)(hp + (int64_t)p * N + n0 + 4);
                bf16x8 v;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    v[e] = (bf16)a0[e];
                    v[e + 4] = (bf16)a1[e];
                }
                *(bf16x8 *)(hs + p * HLD + n0) = v;
            }
        }
    }
    __syncthreads();

    const int T16 = (q + 15) / 16;
    for (int round = 0;; ++round) {
        const int I = 4 * round + ((round & 1) ? 3 - wave : wave);
        if (4 * round >= T16) break;
        if (I >= T16) continue;
        const int il = I * 16 + r;  // this lane's output row inside the chunk
        const bool vi = il < q;
        const float csi = cs_s[il];
        f32x4 acc[PT];
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) acc[pt] = f32x4{0.f, 0.f, 0.f, 0.f};

        const T *crow = Cb + (int64_t)il * G * N;
        // bf16: this tile's C row pieces and C B^T row pieces load in one round,
        // unconditionally (rows past q clamped, values then zeroed), so no
        // branch makes each wait for the one before
        constexpr int NKC = (N + 31) / 32;
        u32x4 cpc[NKC], gpc[8];
        if constexpr (sizeof(T) == 2) {
            const T *crc = Cb + (int64_t)min(il, q - 1) * G * N;
#pragma unroll
            for (int kc = 0; kc < NKC; ++kc) {
                const int kk = kc * 32 + grp * 8;
                cpc[kc] = *(const u32x4 *)(crc + (kk < N ? kk : 0));
            }
            // il < Q: a row of this chunk's tiles; pieces past the row are
            // clamped to its last 8 columns (only pieces with jl <= il are used,
            // and those lie at or before Q - 8)
            const T *grw = cbc + (int64_t)il * Q;
#pragma unroll
            for (int J = 0; J < 8; ++J) gpc[J] = *(const u32x4 *)(grw + min(32 * J + grp * 8, Q - 8));
        }
        if (hp) {
            if constexpr (sizeof(T) == 2) {
#pragma unroll
                for (int kc = 0; kc < NKC; ++kc) {
                    const int kk = kc * 32 + grp * 8;
                    const u32x4 z = {0u, 0u, 0u, 0u};
                    const bf16x8 bcv = as_bf16x8((vi && kk < N) ? cpc[kc] : z);
#pragma unroll
                    for (int pt = 0; pt < PT; ++pt) {
                        const bf16x8 ah =
                            kk < N ? *(const bf16x8 *)(hs + (pt * 16 + r) * HLD + kk) : as_bf16x8(z);
                        acc[pt] = mfma_bf16(ah, bcv, acc[pt]);
                    }
                }
            } else {
                for (int k0 = 0; k0 < N; k0 += 16) {
                    const int kk = k0 + grp * 4;
                    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
                    const f32x4 c4 = vi ? *(const f32x4 *)(crow + kk) : z;
#pragma unroll
                    for (int pt = 0; pt < PT; ++pt) {
                        const f32x4 h4 = *(const f32x4 *)(hp + (int64_t)(pt * 16 + r) * N + kk);
#pragma unroll
                        for (int e = 0; e < 4; ++e) acc[pt] = mfma_f32(h4[e], c4[e], acc[pt]);
                    }
                }
            }
            const float ei = __expf(csi);
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) acc[pt] *= ei;
        }

        const T *grow = cbc + (int64_t)il * Q;
        const int jend = I * 16 + 15;
        if constexpr (sizeof(T) == 2) {
#pragma unroll
            for (int J = 0; J < 8; ++J) {
                const int j0 = 32 * J;
                if (j0 > jend) break;
                const int jl = j0 + grp * 8;
                bf16x8 bm;
                if (jl <= il) {
                    const bf16x8 gv = as_bf16x8(gpc[J]);
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int j = jl + e;
                        const float m = (j <= il) ? __expf(csi - cs_s[j]) * (float)gv[e] * sc_s[j] : 0.f;
                        bm[e] = (bf16)m;
                    }
                } else {
                    bm = as_bf16x8(u32x4{0u, 0u, 0u, 0u});
                }
#pragma unroll
                for (int pt = 0; pt < PT; ++pt) {
                    const bf16x8 ax = *(const bf16x8 *)(xs + (pt * 16 + r) * XLD + jl);
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
                    m[e] = (j <= il) ? __expf(csi - cs_s[j]) * g4[e] * sc_s[j] : 0.f;
                }
#pragma unroll
                for (int pt = 0; pt < PT; ++pt) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int j = jl + e;
                        const float xa = j < q ? to_f32(x[(row0 + (int64_t)j * H) * P + pt * 16 + r]) : 0.f;
                        acc[pt] = mfma_f32(xa, m[e], acc[pt]);
                    }
                }
            }
        }

        if (vi) {
            const T *xr = x + (row0 + (int64_t)il * H) * P;
            T *yr = y + (row0 + (int64_t)il * H) * P;
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) {
                const int p0 = pt * 16 + 4 * grp;
                if constexpr (sizeof(T) == 2) {
                    const u32x2 xw = *(const u32x2 *)(xr + p0);
                    const bf16 *xe = (const bf16 *)&xw;
                    bf16 o[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) o[e] = (bf16)(acc[pt][e] + Dh * (float)xe[e]);
                    *(u32x2 *)(yr + p0) = *(const u32x2 *)o;
                } else {
                    const f32x4 xv = *(const f32x4 *)(xr + p0);
                    *(f32x4 *)(yr + p0) = acc[pt] + Dh * xv;
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// float32 chunk state and output, with the chunk's rows staged in LDS as they
// lie in memory ([j][col], row stride COLS + 4 floats).  The fp32 MFMA takes
// one value per lane: lanes r = 0..15 of a k-group read 16 consecutive
// columns of one row, and the four k-groups read rows 4 apart, which the
// padding of 4 floats puts on the two halves of the 32 banks.  Lane group
// grp of the e-th MFMA of a 16-step block j0 contracts step j0 + 4 grp + e.
// Every global load is unconditional: rows past q are clamped to row q - 1
// and their values replaced by zero, so no branch splits the compiler's
// counted waits.
// ---------------------------------------------------------------------------

// Chunk state S^T[n][p] = sum_j B[j][n] w_j x[j][p] in 64-step slabs: the
// next slab's rows load into registers while the current one is multiplied.
template <int P, int N, bool FROM_START>
__global__ __launch_bounds__(256) void k_chunk_state_f32(const float *__restrict__ x,
                                                         const float *__restrict__ B,
                                                         const float *__restrict__ cs,
                                                         float *__restrict__ S, int64_t L, int H,
                                                         int G, int Q, int nc,
                                                         const float *__restrict__ sc) {
    constexpr int PT = P / 16, NT = N / 16, NTW = (NT + 3) / 4;
    constexpr int SL = 64, XLD = P + 4, BLD = N + 4;
    constexpr int XPC = P / 4, BPC = N / 4;            // 16-byte pieces per row
    constexpr int XPT = SL * XPC / 256, BPT = SL * BPC / 256;  // pieces per thread
    const int64_t wid = xcd_remap(blockIdx.x, gridDim.x);
    const int h = (int)(wid % H);
    const int64_t bc = wid / H;
    const int c = (int)(bc % nc);
    const int64_t b = bc / nc;
    const int g = h / (H / G);
    const int64_t s = (int64_t)c * Q;
    const int q = (int)min<int64_t>(Q, L - s);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int r = lane & 15, grp = lane >> 4;

    __shared__ float w_s[256];
    __shared__ float xs[SL * XLD];
    __shared__ float bs[SL * BLD];
    const float *csc = cs + (((int64_t)b * H + h) * nc + c) * Q;
    const float cs_last = csc[q - 1];
    const float *scc = sc ? sc + (((int64_t)b * H + h) * nc + c) * Q : nullptr;
    for (int j = tid; j < Q; j += 256)
        w_s[j] = (FROM_START ? __expf(csc[j]) : __expf(cs_last - csc[j])) * (scc ? scc[j] : 1.f);

    const float *xb = x + ((b * L + s) * H + h) * P;
    const float *Bb = B + ((b * L + s) * G + g) * N;
    const int64_t xld = (int64_t)H * P, bld = (int64_t)G * N;
    f32x4 xr[XPT], br[BPT];
    auto load = [&](int jb) {
#pragma unroll
        for (int k = 0; k < XPT; ++k) {
            const int idx = tid + 256 * k, j = jb + idx / XPC;
            xr[k] = *(const f32x4 *)(xb + min(j, q - 1) * xld + 4 * (idx % XPC));
        }
#pragma unroll
        for (int k = 0; k < BPT; ++k) {
            const int idx = tid + 256 * k, j = jb + idx / BPC;
            br[k] = *(const f32x4 *)(Bb + min(j, q - 1) * bld + 4 * (idx % BPC));
        }
    };
    // x rows scaled by w_j; rows past q as zero
    auto write = [&](int jb) {
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < XPT; ++k) {
            const int idx = tid + 256 * k, jr = idx / XPC;
            *(f32x4 *)(xs + jr * XLD + 4 * (idx % XPC)) = jb + jr < q ? xr[k] * w_s[jb + jr] : z;
        }
#pragma unroll
        for (int k = 0; k < BPT; ++k) {
            const int idx = tid + 256 * k, jr = idx / BPC;
            *(f32x4 *)(bs + jr * BLD + 4 * (idx % BPC)) = jb + jr < q ? br[k] : z;
        }
    };

    f32x4 acc[NTW][PT];
#pragma unroll
    for (int t = 0; t < NTW; ++t)
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) acc[t][pt] = f32x4{0.f, 0.f, 0.f, 0.f};
    load(0);
    __syncthreads();  // w_s
    for (int jb = 0; jb < q; jb += SL) {
        write(jb);
        lds_barrier();
        load(jb + SL);  // past the end: clamped rows, never written
#pragma unroll
        for (int j0 = 0; j0 < SL; j0 += 16) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int jr = j0 + 4 * grp + e;
                float xa[PT];
#pragma unroll
                for (int pt = 0; pt < PT; ++pt) xa[pt] = xs[jr * XLD + pt * 16 + r];
#pragma unroll
                for (int t = 0; t < NTW; ++t) {
                    const int nt = wave + 4 * t;
                    // (no branch when every wave has NTW tiles: the LDS reads then
                    // run ahead of the MFMAs instead of waiting in each branch)
                    if (NT % 4 == 0 || nt < NT) {
                        const float bv = bs[jr * BLD + nt * 16 + r];
#pragma unroll
                        for (int pt = 0; pt < PT; ++pt) acc[t][pt] = mfma_f32(bv, xa[pt], acc[t][pt]);
                    }
                }
            }
        }
        lds_barrier();
    }
    // acc[t][pt][e] = S^T[n = nt*16 + 4 grp + e][p = pt*16 + r]
    float *So = S + (((b * nc + c) * H + h) * (int64_t)P) * N;
#pragma unroll
    for (int t = 0; t < NTW; ++t) {
        const int nt = wave + 4 * t;
        if (nt < NT) {
#pragma unroll
            for (int pt = 0; pt < PT; ++pt)
                *(f32x4 *)(So + (int64_t)(pt * 16 + r) * N + nt * 16 + 4 * grp) = acc[t][pt];
        }
    }
}

// Output of a chunk, transposed as in k_chunk_scan: Y^T[p][i] per 16-row
// tile, the waves' tiles dealt in the same snake order.  The state term runs
// first for all four of a wave's tiles, so h_{c-1} is read once per wave;
// each tile's C B^T row pieces load in one round (buffer loads, the blocks
// past the diagonal switched off) before its intra product.  Every tile is
// computed, a tile past q on clamped rows; its stores fall outside the
// buffer resource over y and are dropped.  The next tile's C B^T pieces load
// while a tile computes.  The caller keeps the byte span
// of a chunk's y rows below 2^31.
template <int P, int N>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_chunk_scan_f32(const float *__restrict__ x,
                                                        const float *__restrict__ C,
                                                        const float *__restrict__ cb,
                                                        const float *__restrict__ cs,
                                                        const float *__restrict__ hprev,
                                                        const float *__restrict__ D,
                                                        float *__restrict__ y, int64_t L, int H,
                                                        int G, int Q, int nc,
                                                        const float *__restrict__ sc) {
    constexpr int PT = P / 16, XLD = P + 4, PC = P / 4, KB = PC < 8 ? PC : 8;
    const int64_t wid = xcd_remap(blockIdx.x, gridDim.x);
    const int h = (int)(wid % H);
    const int64_t bc = wid / H;
    const int c = (int)(bc % nc);
    const int64_t b = bc / nc;
    const int g = h / (H / G);
    const int64_t s = (int64_t)c * Q;
    const int q = (int)min<int64_t>(Q, L - s);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int r = lane & 15, grp = lane >> 4;

    __shared__ float cs_s[256], sc_s[256];
    __shared__ float xs[256 * XLD];
    const float *csc = cs + (((int64_t)b * H + h) * nc + c) * Q;
    const float *scc = sc ? sc + (((int64_t)b * H + h) * nc + c) * Q : nullptr;
    cs_s[tid] = csc[min(tid, Q - 1)];
    sc_s[tid] = scc ? scc[min(tid, Q - 1)] : 1.f;
    const int64_t row0 = (b * L + s) * H + h;  // (row of step s, head h) in x / y
    const int64_t HP = (int64_t)H * P;
    const float *xb = x + row0 * P;
    // the chunk's x rows, rows q .. 255 as zero
#pragma unroll
    for (int k0 = 0; k0 < PC; k0 += KB) {
        f32x4 v[KB];
#pragma unroll
        for (int k = 0; k < KB; ++k) {
            const int idx = tid + 256 * (k0 + k);
            v[k] = *(const f32x4 *)(xb + min(idx / PC, q - 1) * HP + 4 * (idx % PC));
        }
#pragma unroll
        for (int k = 0; k < KB; ++k) {
            const int idx = tid + 256 * (k0 + k), j = idx / PC;
            *(f32x4 *)(xs + j * XLD + 4 * (idx % PC)) = j < q ? v[k] : f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }
    __syncthreads();

    const float *cbc = cb + (((int64_t)b * nc + c) * G + g) * (int64_t)Q * Q;
    const float *hp = hprev ? hprev + (((b * nc + c) * H + h) * (int64_t)P) * N : nullptr;
    const float *Cb = C + ((b * L + s) * G + g) * N;
    const int64_t GN = (int64_t)G * N;
    const float Dh = D ? D[h] : 0.f;
    int tI[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) tI[t] = 4 * t + ((t & 1) ? 3 - wave : wave);
    // tiles past Q (Q < 256) are computed on clamped rows and never stored
    f32x4 acc[4][PT];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) acc[t][pt] = f32x4{0.f, 0.f, 0.f, 0.f};

    // C B^T row pieces of tile t's blocks 0..I (the rest read as zero), in two
    // register sets used in turn: tile t + 1's load while tile t computes
    const auto rsG = buf_rsrc(cbc, (uint32_t)Q * (uint32_t)Q * 4u);
    f32x4 gA[16], gB[16];
    auto load_g = [&](int t, f32x4(&g4)[16]) {
        const int I = tI[t], ilc = min(I * 16 + r, q - 1);
#pragma unroll
        for (int jb = 0; jb < 16; ++jb)
            g4[jb] = __builtin_bit_cast(
                f32x4, buf_ld16(rsG, jb <= I && jb * 16 < Q ? (uint32_t)(ilc * Q + jb * 16 + 4 * grp) * 4u : kBufOff));
    };
    load_g(0, gA);

    // state term exp(cs_i) C_i h_{c-1}: A = h rows, B = C rows; the pieces of
    // step k + 1 load while step k multiplies (two register sets)
    if (hp) {
        constexpr int NK = N / 16;
        f32x4 h4[2][PT], c4[2][4];
        auto load_hc = [&](int k, f32x4(&hv)[PT], f32x4(&cv)[4]) {
            const int kk = k * 16 + 4 * grp;
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) hv[pt] = *(const f32x4 *)(hp + (int64_t)(pt * 16 + r) * N + kk);
#pragma unroll
            for (int t = 0; t < 4; ++t) cv[t] = *(const f32x4 *)(Cb + min(tI[t] * 16 + r, q - 1) * GN + kk);
        };
        load_hc(0, h4[0], c4[0]);
#pragma unroll
        for (int k = 0; k < NK; ++k) {
            if (k + 1 < NK) load_hc(k + 1, h4[(k + 1) & 1], c4[(k + 1) & 1]);
            __builtin_amdgcn_sched_barrier(0);  // the prefetch stays ahead of the MFMAs
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int pt = 0; pt < PT; ++pt)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        acc[t][pt] = mfma_f32(h4[k & 1][pt][e], c4[k & 1][t][e], acc[t][pt]);
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const float ei = __expf(cs_s[tI[t] * 16 + r]);
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) acc[t][pt] *= ei;
        }
    }

    const auto rsY = buf_rsrc(y + row0 * P, (uint32_t)(((int64_t)(q - 1) * HP + P) * 4));
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        f32x4(&g4)[16] = (t & 1) ? gB : gA;
        if (t + 1 < 4) load_g(t + 1, (t & 1) ? gA : gB);  // the next tile's, in flight meanwhile
        __builtin_amdgcn_sched_barrier(0);
        const int I = tI[t];
        const int il = I * 16 + r;  // this lane's output row inside the chunk
        const float csi = cs_s[il];
#pragma unroll
        for (int jb = 0; jb < 16; ++jb) {
            if (jb <= I) {
                const int jl = jb * 16 + 4 * grp;
                const f32x4 csj = *(const f32x4 *)(cs_s + jl), scj = *(const f32x4 *)(sc_s + jl);
                float m[4];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    m[e] = (jl + e <= il) ? __expf(csi - csj[e]) * g4[jb][e] * scj[e] : 0.f;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
#pragma unroll
                    for (int pt = 0; pt < PT; ++pt)
                        acc[t][pt] = mfma_f32(xs[(jl + e) * XLD + pt * 16 + r], m[e], acc[t][pt]);
                }
            }
        }
        // + D x_i; lane holds row il, channels p0 .. p0 + 3
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) {
            const int p0 = pt * 16 + 4 * grp;
            const f32x4 o = acc[t][pt] + Dh * *(const f32x4 *)(xs + il * XLD + p0);
            const uint32_t off = il < q ? (uint32_t)((il * HP + p0) * 4) : kBufOff;
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, o), rsY, (int)off, 0, 0);
        }
    }
}

// ---------------------------------------------------------------------------
// Decode step: one workgroup per (b, h).  N / 4 lanes share a state row (one
// float4 each); rows are processed 8 deep so 8 loads per lane are in flight.
// The row dot product with C is a butterfly over the row's lanes.
// ---------------------------------------------------------------------------
template <typename T, int N>
__global__ __launch_bounds__(256) void k_decode(float *__restrict__ state, const T *__restrict__ x,
                                                const T *__restrict__ dt,
                                                const float *__restrict__ A,
                                                const T *__restrict__ B, const T *__restrict__ C,
                                                const float *__restrict__ D, T *__restrict__ y,
                                                int H, int G, int P, DtOpts o, int use_opts) {
    constexpr int NL = N / 4, RPI = 256 / NL, U = 8;
    const int64_t bh = blockIdx.x;
    const int h = (int)(bh % H);
    const int64_t b = bh / H;
    const int g = h / (H / G);
    const int nl = threadIdx.x % NL, slot = threadIdx.x / NL;
    const float dte = use_opts ? dt_effective(to_f32(dt[bh]), h, o) : to_f32(dt[bh]);
    const float a = __expf(dte * A[h]);
    const float xsc = use_opts ? input_scale(dte, A[h], o.scale) : 1.f;  // x's factor in the update
    const float Dh = D ? D[h] : 0.f;
    float bv[4], cv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        bv[e] = to_f32(B[(b * G + g) * N + nl * 4 + e]);
        cv[e] = to_f32(C[(b * G + g) * N + nl * 4 + e]);
    }
    float *st = state + bh * (int64_t)P * N;
    const T *xp = x + bh * P;
    T *yp = y + bh * P;
    // Loads are unconditional (rows past P clamped to row P - 1) and stores go
    // through buffer resources whose switched-off lanes point past the end, so
    // no branch makes the compiler wait for each load, or each store, in turn.
    // The state streams through once per step: non-temporal accesses.
    const auto rsS = buf_rsrc(st, (uint32_t)P * N * 4u);
    const auto rsY = buf_rsrc(yp, (uint32_t)P * (uint32_t)sizeof(T));
    for (int p0 = 0; p0 < P; p0 += RPI * U) {
        f32x4 hv[U];
        T xr[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int pc = min(p0 + u * RPI + slot, P - 1);
            hv[u] = __builtin_nontemporal_load((const f32x4 *)(st + (int64_t)pc * N + nl * 4));
            xr[u] = xp[pc];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int p = p0 + u * RPI + slot;
            const float xv = to_f32(xr[u]);
            float part = 0.f;
            f32x4 nh;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                nh[e] = a * hv[u][e] + (xsc * xv) * bv[e];
                part += nh[e] * cv[e];
            }
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, nh), rsS,
                                                   p < P ? (p * N + nl * 4) * 4 : (int)kBufOff, 0, 2);
#pragma unroll
            for (int off = NL / 2; off >= 1; off >>= 1) part += __shfl_xor(part, off, 64);
            const int yo = (nl == 0 && p < P) ? p * (int)sizeof(T) : (int)kBufOff;
            const T yv = from_f32<T>(part + Dh * xv);
            if constexpr (sizeof(T) == 2)
                __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, yv), rsY, yo, 0, 0);
            else
                __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, yv), rsY, yo, 0, 0);
        }
    }
}

// ---------------------------------------------------------------------------
// Decode step over "pieces" (used when RPI = 256 / (N / 4) divides P).  The
// state rows of all (b, h) slices form one array of nbh * P rows of N floats
// (x and y: nbh * P values); a piece is RPI consecutive rows of one slice,
// one float4 per lane.  The grid strides over pieces, U pieces per lane in
// flight, consecutive workgroups on consecutive pieces, so the workgroups
// resident at one time stream one contiguous window of the array (on MI355X
// this moves the state 2-6% faster than one whole slice per workgroup, and
// as fast as a plain non-temporal read-modify-write of the same bytes).  A
// piece's slice, and with it dt, A, D, is uniform over the workgroup (scalar
// loads); B and C rows come in one vector load per lane.
// ---------------------------------------------------------------------------
template <typename T> struct Raw4;  // four consecutive elements, one load
template <> struct Raw4<bf16> { using type = uint2; };
template <> struct Raw4<float> { using type = f32x4; };

template <typename T>
__device__ __forceinline__ float raw4_at(const typename Raw4<T>::type &v, int e) {
    if constexpr (sizeof(T) == 2) {
        const uint32_t w = e < 2 ? v.x : v.y;
        return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
    } else {
        return v[e];
    }
}

template <typename T, int N, int U>
__global__ __launch_bounds__(256) void k_decode_pieces(
    float *__restrict__ state, const T *__restrict__ x, const T *__restrict__ dt,
    const float *__restrict__ A, const T *__restrict__ B, const T *__restrict__ C,
    const float *__restrict__ D, T *__restrict__ y, int npieces, int pps_log2, int H, int G,
    DtOpts o, int use_opts) {
    constexpr int NL = N / 4, RPI = 256 / NL;
    using R4 = typename Raw4<T>::type;
    const int nl = threadIdx.x % NL, slot = threadIdx.x / NL;
    const int gs = (int)gridDim.x;
    // Workgroups are dealt to the 8 XCDs in turn.  Within each run of 64
    // workgroups, swap the two 3-bit digits of the index, so that XCD x takes
    // pieces 8x .. 8x + 7 of the run's 64: a slice's neighbouring pieces
    // (which share x and y cache lines) stay in one L2, and the run still
    // covers 64 consecutive pieces.  Needs a grid that is a multiple of 64.
    const int w = (int)blockIdx.x;
    const int wq = (gs & 63) == 0 ? ((w & ~63) | ((w & 7) << 3) | ((w >> 3) & 7)) : w;
    for (int q0 = wq; q0 < npieces; q0 += U * gs) {
        f32x4 hv[U];
        R4 bv[U], cv[U];
        T xr[U];
        float av[U], sv[U], dv[U];
        // all loads first and unconditional: a slot past the end re-reads
        // this pass's first piece and stores nothing (re-reading one shared
        // piece instead would send every workgroup to the same addresses)
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int q = q0 + u * gs < npieces ? q0 + u * gs : q0;
            const int bh = q >> pps_log2;
            const int h = bh % H, g = h / (H / G);
            const int64_t bg = (int64_t)(bh / H) * G + g;
            const int64_t r = (int64_t)q * RPI + slot;
            hv[u] = __builtin_nontemporal_load((const f32x4 *)(state + r * N + nl * 4));
            xr[u] = x[r];
            bv[u] = *(const R4 *)(B + bg * N + nl * 4);
            cv[u] = *(const R4 *)(C + bg * N + nl * 4);
            const float dte = use_opts ? dt_effective(to_f32(dt[bh]), h, o) : to_f32(dt[bh]);
            av[u] = __expf(dte * A[h]);
            sv[u] = use_opts ? input_scale(dte, A[h], o.scale) : 1.f;  // x's factor in the update
            dv[u] = D ? D[h] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int q = q0 + u * gs;
            if (q >= npieces) break;  // uniform
            const int64_t r = (int64_t)q * RPI + slot;
            const float xv = to_f32(xr[u]);
            float part = 0.f;
            f32x4 nh;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                nh[e] = av[u] * hv[u][e] + (sv[u] * xv) * raw4_at<T>(bv[u], e);
                part += nh[e] * raw4_at<T>(cv[u], e);
            }
            __builtin_nontemporal_store(nh, (f32x4 *)(state + r * N + nl * 4));
#pragma unroll
            for (int off = NL / 2; off >= 1; off >>= 1) part += __shfl_xor(part, off, 64);
            if (nl == 0) y[r] = from_f32<T>(part + dv[u] * xv);
        }
    }
}

// ---------------------------------------------------------------------------
// Launchers.
// ---------------------------------------------------------------------------
#define SSD_DISPATCH_PN(P_, N_, ...)                                              \
    do {                                                                          \
        switch (P_) {                                                             \
        case 16: { constexpr int PP = 16; SSD_DISPATCH_N(N_, __VA_ARGS__); } break; \
        case 32: { constexpr int PP = 32; SSD_DISPATCH_N(N_, __VA_ARGS__); } break; \
        case 64: { constexpr int PP = 64; SSD_DISPATCH_N(N_, __VA_ARGS__); } break; \
        case 128: { constexpr int PP = 128; SSD_DISPATCH_N(N_, __VA_ARGS__); } break; \
        default: return hipErrorInvalidValue;                                     \
        }                                                                         \
    } while (0)
#define SSD_DISPATCH_N(N_, ...)                                                   \
    switch (N_) {                                                                 \
    case 16: { constexpr int NN = 16; __VA_ARGS__; } break;                       \
    case 32: { constexpr int NN = 32; __VA_ARGS__; } break;                       \
    case 64: { constexpr int NN = 64; __VA_ARGS__; } break;                       \
    case 128: { constexpr int NN = 128; __VA_ARGS__; } break;                     \
    case 256: { constexpr int NN = 256; __VA_ARGS__; } break;                     \
    default: return hipErrorInvalidValue;                                         \
    }

hipError_t launch_chunk_cumsum(const Dims &d, const void *dt, const float *A, float *cs,
                               hipStream_t st) {
    if (d.b == 0 || d.nc == 0) return hipSuccess;
    dim3 grid((unsigned)d.nc, (unsigned)d.H, (unsigned)d.b);
    if (d.dtype == 1)
        k_chunk_cumsum<bf16><<<grid, 64, 0, st>>>((const bf16 *)dt, A, cs, d.L, (int)d.H, (int)d.Q,
                                                  (int)d.nc);
    else
        k_chunk_cumsum<float><<<grid, 64, 0, st>>>((const float *)dt, A, cs, d.L, (int)d.H,
                                                   (int)d.Q, (int)d.nc);
    return hipGetLastError();
}

hipError_t launch_chunk_cumsum_opts(const Dims &d, const void *dt, const float *A,
                                    const DtOpts &o, float *cs, float *sc, hipStream_t st) {
    if (d.b == 0 || d.nc == 0) return hipSuccess;
    dim3 grid((unsigned)d.nc, (unsigned)d.H, (unsigned)d.b);
    if (d.dtype == 1)
        k_chunk_cumsum_opts<bf16><<<grid, 64, 0, st>>>((const bf16 *)dt, A, o, cs, sc, d.L, (int)d.H,
                                                       (int)d.Q, (int)d.nc);
    else
        k_chunk_cumsum_opts<float><<<grid, 64, 0, st>>>((const float *)dt, A, o, cs, sc, d.L,
                                                        (int)d.H, (int)d.Q, (int)d.nc);
    return hipGetLastError();
}

hipError_t launch_chunk_cb(const Dims &d, const void *B, const void *C, void *cb, void *cbT,
                           hipStream_t st) {
    if (d.b == 0 || d.nc == 0) return hipSuccess;
    const int T16 = (int)(d.Q / 16);
    const int ntiles = T16 * (T16 + 1) / 2;
    dim3 grid((unsigned)(d.b * d.nc * d.G), (unsigned)((ntiles + 3) / 4));
    SSD_DISPATCH_N(d.N, {
        if (d.dtype == 1)
            k_chunk_cb<bf16, NN><<<grid, 256, 0, st>>>((const bf16 *)B, (const bf16 *)C, (bf16 *)cb,
                                                       (bf16 *)cbT, d.L, (int)d.G, (int)d.Q, (int)d.nc);
        else
            k_chunk_cb<float, NN><<<grid, 256, 0, st>>>((const float *)B, (const float *)C, (float *)cb,
                                                        (float *)cbT, d.L, (int)d.G, (int)d.Q, (int)d.nc);
    });
    return hipGetLastError();
}

hipError_t launch_chunk_state(const Dims &d, const void *x, const void *B, const float *cs,
                              float *S, bool from_start, hipStream_t st, const float *sc) {
    if (d.b == 0 || d.nc == 0) return hipSuccess;
    if (d.dtype == 1 && (d.P == 32 || d.P == 64) && (d.N == 64 || d.N == 128) && d.Q % 32 == 0) {
        // heads split into parts so that the workgroups fill every CU once
        // (as many per CU as their LDS allows)
        const int64_t nbcg = d.b * d.nc * d.G, hpg = d.H / d.G;
        // workgroups per CU that registers and LDS allow (8-wave workgroups for N = 128
        // need about 176 VGPRs: one per CU; 4-wave ones for N = 64: two)
        const int64_t target = 256 * (d.N == 128 ? 1 : 2);
#define SSD_LAUNCH_STATE_MH(PV, NV)                                                               \
        const int nparts = (int)std::max<int64_t>(1, std::min<int64_t>(hpg, (target + nbcg - 1) / nbcg)); \
        const unsigned g2 = (unsigned)(nbcg * nparts);                                            \
        if (from_start)                                                                           \
            k_chunk_state_mh<PV, NV, true><<<g2, 64 * (NV / 16), 0, st>>>((const bf16 *)x, (const bf16 *)B, cs, S, \
                d.L, (int)d.H, (int)d.G, (int)d.Q, (int)d.nc, sc, nparts);                        \
        else                                                                                      \
            k_chunk_state_mh<PV, NV, false><<<g2, 64 * (NV / 16), 0, st>>>((const bf16 *)x, (const bf16 *)B, cs, S, \
                d.L, (int)d.H, (int)d.G, (int)d.Q, (int)d.nc, sc, nparts);
        if (d.P == 32 && d.N == 64) { SSD_LAUNCH_STATE_MH(32, 64) }
        else if (d.P == 32) { SSD_LAUNCH_STATE_MH(32, 128) }
        else if (d.N == 64) { SSD_LAUNCH_STATE_MH(64, 64) }
        else { SSD_LAUNCH_STATE_MH(64, 128) }
#undef SSD_LAUNCH_STATE_MH
        return hipGetLastError();
    }
    const unsigned grid = (unsigned)(d.b * d.nc * d.H);
#define SSD_LAUNCH_STATE(FS)                                                                      \
    SSD_DISPATCH_PN(d.P, d.N, {                                                                   \
        if (d.dtype == 1)                                                                         \
            k_chunk_state<bf16, PP, NN, FS><<<grid, 256, 0, st>>>(                                \
                (const bf16 *)x, (const bf16 *)B, cs, S, d.L, (int)d.H, (int)d.G, (int)d.Q,       \
                (int)d.nc, sc);                                                                   \
        else                                                                                      \
            k_chunk_state_f32<PP, NN, FS><<<grid, 256, 0, st>>>(                                  \
                (const float *)x, (const float *)B, cs, S, d.L, (int)d.H, (int)d.G, (int)d.Q,     \
                (int)d.nc, sc);                                                                   \
    })
    if (from_start) SSD_LAUNCH_STATE(true);
    else SSD_LAUNCH_STATE(false);
#undef SSD_LAUNCH_STATE
    return hipGetLastError();
}

hipError_t launch_state_passing(const Dims &d, float *S, const float *cs, const float *init,
                                float *fin, hipStream_t st) {
    if (d.b == 0) return hipSuccess;
    const int PN = (int)(d.P * d.N);
    if (d.nc == 0) {
        if (!fin) return hipSuccess;
        const int64_t n = d.b * d.H * PN;
        k_copy_state<<<(unsigned)((n / 4 + 255) / 256), 256, 0, st>>>(init, fin, n);
        return hipGetLastError();
    }
    dim3 grid((unsigned)((PN / 4 + 255) / 256), (unsigned)d.H, (unsigned)d.b);
    k_state_passing<<<grid, 256, 0, st>>>(S, cs, init, fin, d.L, (int)d.H, PN, (int)d.Q,
                                          (int)d.nc);
    return hipGetLastError();
}

hipError_t launch_zero_state(const Dims &d, const float *init, float *fin, hipStream_t st) {
    if (d.b == 0 || !fin) return hipSuccess;
    const int64_t n = d.b * d.H * d.P * d.N;
    k_copy_state<<<(unsigned)((n / 4 + 255) / 256), 256, 0, st>>>(init, fin, n);
    return hipGetLastError();
}

hipError_t launch_chunk_scan(const Dims &d, const void *x, const void *C, const void *cb,
                             const float *cs, const float *hprev, const float *D, void *y,
                             hipStream_t st, const float *sc) {
    if (d.b == 0 || d.nc == 0) return hipSuccess;
    const unsigned grid = (unsigned)(d.b * d.nc * d.H);
    // k_chunk_scan_f32 addresses a chunk's y rows through one buffer resource
    const bool f32_span_ok = d.Q * d.H * d.P * 4 < ((int64_t)1 << 31);
    SSD_DISPATCH_PN(d.P, d.N, {
        if (d.dtype == 1)
            k_chunk_scan<bf16, PP, NN><<<grid, 256, 0, st>>>(
                (const bf16 *)x, (const bf16 *)C, (const bf16 *)cb, cs, hprev, D, (bf16 *)y, d.L,
                (int)d.H, (int)d.G, (int)d.Q, (int)d.nc, sc);
        else if (f32_span_ok)
            k_chunk_scan_f32<PP, NN><<<grid, 256, 0, st>>>(
                (const float *)x, (const float *)C, (const float *)cb, cs, hprev, D, (float *)y,
                d.L, (int)d.H, (int)d.G, (int)d.Q, (int)d.nc, sc);
        else
            k_chunk_scan<float, PP, NN><<<grid, 256, 0, st>>>(
                (const float *)x, (const float *)C, (const float *)cb, cs, hprev, D, (float *)y,
                d.L, (int)d.H, (int)d.G, (int)d.Q, (int)d.nc, sc);
    });
    return hipGetLastError();
}

// Piece decode launch shape: two pieces in flight per lane and at most 81920
// workgroups (one pass over the 256 x 80 x 64 x 128 state).  Measured on
// MI355X with launches back to back and with the caches flushed between them,
// this beat 1, 3 or 4 pieces per lane and grids of 16384 to 65536.
constexpr int kDecodeU = 2;
constexpr int kDecodeGrid = 81920;

hipError_t launch_decode(const Dims &d, float *state, const void *x, const void *dt,
                         const float *A, const void *B, const void *C, const float *D, void *y,
                         hipStream_t st, const DtOpts *o) {
    if (d.b == 0) return hipSuccess;
    const DtOpts oo = o ? *o : DtOpts{nullptr, 0.f, 0.f, 0, 0};
    const int use = o ? 1 : 0;
    const int64_t nrows = d.b * d.H * d.P;
    if (nrows > kDecodeMaxRows) return hipErrorInvalidValue;  // rejected earlier by the ABI layer
    SSD_DISPATCH_N(d.N, {
        constexpr int RPI = 256 / (NN / 4);
        if (d.P % RPI == 0) {
            const int npieces = (int)(nrows / RPI);
            int pl = 0;
            while ((RPI << pl) < d.P) ++pl;  // P / RPI = 2^pl (P and RPI are powers of two)
            int64_t grid = std::min<int64_t>(kDecodeGrid, (npieces + kDecodeU - 1) / kDecodeU);
            if (grid > 64) grid = (grid + 63) / 64 * 64;  // for the XCD-aware order; spare workgroups idle
            if (d.dtype == 1)
                k_decode_pieces<bf16, NN, kDecodeU><<<(unsigned)grid, 256, 0, st>>>(
                    state, (const bf16 *)x, (const bf16 *)dt, A, (const bf16 *)B, (const bf16 *)C, D, (bf16 *)y,
                    npieces, pl, (int)d.H, (int)d.G, oo, use);
            else
                k_decode_pieces<float, NN, kDecodeU><<<(unsigned)grid, 256, 0, st>>>(
                    state, (const float *)x, (const float *)dt, A, (const float *)B, (const float *)C, D, (float *)y,
                    npieces, pl, (int)d.H, (int)d.G, oo, use);
        } else if (d.dtype == 1) {
            k_decode<bf16, NN><<<(unsigned)(d.b * d.H), 256, 0, st>>>(
                state, (const bf16 *)x, (const bf16 *)dt, A, (const bf16 *)B, (const bf16 *)C, D, (bf16 *)y,
                (int)d.H, (int)d.G, (int)d.P, oo, use);
        } else {
            k_decode<float, NN><<<(unsigned)(d.b * d.H), 256, 0, st>>>(
                state, (const float *)x, (const float *)dt, A, (const float *)B, (const float *)C, D, (float *)y,
                (int)d.H, (int)d.G, (int)d.P, oo, use);
        }
    });
    return hipGetLastError();
}

}  // namespace ssd
