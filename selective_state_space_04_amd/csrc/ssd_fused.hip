// Single-pass SSD forward for bfloat16 inputs (gfx950).
//
// One workgroup per (b, c, h) does every step of the chunked algorithm for
// its chunk (Mamba-2 review, docsaid.org, section "2つのルートを半分ずつ":
// the quadratic form inside the block, only the end-of-block state handed to
// the next block), so x is read from HBM once and y is written once:
//   1. decay prefix cs of the chunk (wave scans over dt * A_h)
//   2. x^T staged in LDS
//   3. wait for the state entering the chunk and start loading it
//   4. chunk state S_c^T = sum_j (w_j B_j)^T x_j, w_j = exp(cs_last - cs_j)
//   5. h_c = exp(cs_last) h_{c-1} + S_c handed to chunk c + 1 (or written as
//      final_state); h_{c-1} kept in LDS for step 6
//   6. y = (C B^T masked by exp(cs_i - cs_j) [j <= i]) x + exp(cs_i) C_i h_{c-1}
//      + D x_i, per 16-row output tile
// A preparation kernel writes C B^T, B^T and C of every chunk in MFMA-fragment
// order beforehand (they are shared by all heads of a group).
//
// Every factor exp(a) used in the factorised mask has a <= 0 (cs is
// non-increasing for dt >= 0, A <= 0), so nothing overflows; a factor that
// underflows multiplies a contribution that is itself below the float range.
//
// Ordering: block ids map to (c, b, h) so that the workgroup chunk c waits
// on always has a smaller id in the same dispatch stream; with in-order
// dispatch it is already resident or done, so the chain always drains.  The
// wait is also bounded (it gives up after ~0.1 s and the result is then
// wrong, never hung).  The handed-off state is written and read with
// agent-scope atomic accesses, which are coherent across the XCDs' separate
// L2 caches.  Each wave hands off its own slice of the state: it raises its
// flag only after its slice's stores have completed (s_waitcnt), and the
// reading wave issues its loads only after it has seen that flag.
#include <type_traits>

#include "ssd_device.h"
#include "ssd_launch.h"

namespace ssd {

namespace {

constexpr int kSpinLimit = 1 << 21;

// 16-byte ring load / store carrying the SC1 cache-policy bit (operand 16),
// which is what the compiler emits for an agent-scope relaxed atomic load or
// store on gfx950: coherent across the XCDs' separate L2 caches with no
// cache write-back/invalidate, at twice the width of a 64-bit atomic.
constexpr int kAgentCoherent = 16;
__device__ __forceinline__ f32x4 ld_agent_f32x4(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)off, 0, kAgentCoherent));
}
__device__ __forceinline__ void st_agent_f32x4(f32x4 v, __amdgpu_buffer_rsrc_t rs, uint32_t off) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rs, (int)off, 0, kAgentCoherent);
}

// x staging, split so the loads can be issued long before the LDS writes.
// A thread owns up to XB blocks of 4 rows x 8 columns: blocks tid, tid + 256.
template <int P>
struct XStage {
    static constexpr int NBC = P / 8;                  // 8-column blocks per row group
    static constexpr int XB = (256 / 4) * NBC / 256;   // blocks per thread for 256 rows
    u32x4 v[XB][4];
};

// Block blk -> (row group br, column block bc).  Each 32-lane half-wave
// covers 16 consecutive row groups and two adjacent column blocks, so its
// transposed 8-byte LDS stores hit distinct banks.  (Eight adjacent lanes
// per row would read whole rows, but their transposed stores then collide
// eight ways, which costs more.)
template <int P>
__device__ __forceinline__ void xstage_block(int blk, int &br, int &bc) {
    constexpr int NBC = XStage<P>::NBC;
    bc = (blk >> 4) % NBC;
    br = (blk & 15) + 16 * ((blk >> 4) / NBC);
}

// LDS tiles with rows of 16-byte chunks, unpadded; chunk k of row `row` is
// stored at k ^ (row & 15).  A 16-byte operand read by lanes r = 0..15
// (rows 16 pt + r) at chunk 4 J + grp then covers all banks once, and so do
// the transposed staging stores.  Offsets in elements; W = row length.
template <int W>
__device__ __forceinline__ int swz(int row, int col) {
    return row * W + ((((col >> 3) ^ row) & 15) | ((col >> 3) & ~15)) * 8 + (col & 7);
}

template <int P>
__device__ __forceinline__ void stage_x_load(XStage<P> &st, const bf16 *__restrict__ src, int ld,
                                             int nvalid) {
    // x is read once: a non-temporal load (cache policy bit 1) keeps it from
    // displacing the per-chunk operands every head of the chunk re-reads.
    // Rows past nvalid read as zero: their lanes are given an offset past the
    // resource's end, so no load sits behind a branch.
    const auto rs = buf_rsrc(src, (uint32_t)nvalid * (uint32_t)ld * 2u);
#pragma unroll
    for (int i = 0; i < XStage<P>::XB; ++i) {
        int br, bc;
        xstage_block<P>(threadIdx.x + 256 * i, br, bc);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int rr = br * 4 + k;
            st.v[i][k] = __builtin_amdgcn_raw_buffer_load_b128(
                rs, (int)(rr < nvalid ? ((uint32_t)rr * ld + bc * 8) * 2u : kBufOff), 0, 2);
        }
    }
}

// Write the loaded blocks transposed into the chunk-swizzled x^T tile
// (row = column of x, 256 steps per row); rows past q were loaded as zero.
template <int P>
__device__ __forceinline__ void stage_x_write_swz(const XStage<P> &st, bf16 *xs) {
#pragma unroll
    for (int i = 0; i < XStage<P>::XB; ++i) {
        int br, bc;
        xstage_block<P>(threadIdx.x + 256 * i, br, bc);
        const int r0 = br * 4, c0 = bc * 8;
        const u32x4 *v = st.v[i];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            *(u32x2 *)(xs + swz<256>(c0 + 2 * m, r0)) =
                u32x2{__builtin_amdgcn_perm(v[1][m], v[0][m], 0x05040100u),
                      __builtin_amdgcn_perm(v[3][m], v[2][m], 0x05040100u)};
            *(u32x2 *)(xs + swz<256>(c0 + 2 * m + 1, r0)) =
                u32x2{__builtin_amdgcn_perm(v[1][m], v[0][m], 0x07060302u),
                      __builtin_amdgcn_perm(v[3][m], v[2][m], 0x07060302u)};
        }
    }
}

}  // namespace

// ---------------------------------------------------------------------------
// Preparation for the single-pass kernel.  It writes the operands shared by
// all heads of a group in MFMA-fragment order, so the single-pass kernel
// loads each fragment of a wave as one contiguous 1 KiB block (lane l of the
// fragment at byte 16 l).  For chunk (b, c, g), with r = l % 16, q4 = l / 16:
//   Gf [I][J][l]  = C B^T rows 16 I + r, columns 32 J + 8 q4 .. + 7
//                   (I < Q/16, J <= I/2; the diagonal 32-block is complete)
//   Btf[t][J][l]  = B rows 32 J + 8 q4 .. + 7 at column 16 t + r  (B^T)
//   Cf [I][k][l]  = C row 16 I + r, columns 32 k + 8 q4 .. + 7
// Rows past the sequence end are zero.  One workgroup per 64 x 64 block
// (bi, bj), bj <= bi, of C B^T: it stages C rows 64 bi .. + 63 and B rows
// 64 bj .. + 63 in LDS (whole-row loads) and wave w computes row tile
// 4 bi + w.  Diagonal blocks also write the C fragments of their rows and
// the B^T fragments of their 32-blocks; block (0, 0) clears the flags.
// ---------------------------------------------------------------------------
template <int N>
__global__ __launch_bounds__(256) void k_fused_prep(const bf16 *__restrict__ B,
                                                    const bf16 *__restrict__ C,
                                                    bf16 *__restrict__ Gf, bf16 *__restrict__ Btf,
                                                    bf16 *__restrict__ Cf, int *flags, int nflags,
                                                    int L, int G, int Q, int nc) {
    constexpr int NKN = N / 32, NTT = N / 16;
    constexpr int RLD = N + 8;            // LDS row stride (elements): 16-byte reads spread over banks
    constexpr int RCH = N / 8;            // 16-byte pieces per row
    __shared__ bf16 cs_rows[64 * RLD];
    __shared__ bf16 bs_rows[64 * RLD];
    const int T16 = Q / 16, NJ = (Q + 31) / 32;
    const int bcg = blockIdx.x;
    const int g = bcg % G;
    const int bc = bcg / G;
    const int c = bc % nc;
    const int b = bc / nc;
    const int s = c * Q;
    const int q = min(Q, L - s);
    // block (bi, bj) from the lower-triangular index
    int bi = 0, bj = blockIdx.y;
    while (bj > bi) {
        bj -= bi + 1;
        ++bi;
    }
    const bool diag = bi == bj;
    const bf16 *Bc = B + ((int64_t)(b * L + s) * G + g) * N;
    const bf16 *Cc = C + ((int64_t)(b * L + s) * G + g) * N;
    const int ld = G * N;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int r = lane & 15, grp = lane >> 4;
    const u32x4 z = {0u, 0u, 0u, 0u};
    if (diag && bi == 0 && bcg == 0)
        for (int i = tid; i < nflags; i += 256) flags[i] = 0;

    // stage: 64 C rows and 64 B rows, RCH adjacent lanes per row (rows past q: zero)
    for (int it = tid; it < 64 * RCH; it += 256) {
        const int row = it / RCH, ch = it % RCH;
        const int ci = 64 * bi + row, bj_row = 64 * bj + row;
        const u32x4 vc = ci < q ? *(const u32x4 *)(Cc + (int64_t)ci * ld + ch * 8) : z;
        const u32x4 vb = bj_row < q ? *(const u32x4 *)(Bc + (int64_t)bj_row * ld + ch * 8) : z;
        *(u32x4 *)(cs_rows + row * RLD + ch * 8) = vc;
        *(u32x4 *)(bs_rows + row * RLD + ch * 8) = vb;
    }
    __syncthreads();

    const int I = 4 * bi + wave;  // row tile of this wave
    if (I < T16) {
        // C B^T tiles (I, jt), jt = 4 bj .. 4 bj + 3, computed transposed so each
        // lane holds four consecutive columns j of one row i:
        // D[m = j][n = i] = sum_k B_j C_i
        bf16x8 cf[NKN];
#pragma unroll
        for (int k = 0; k < NKN; ++k)
            cf[k] = *(const bf16x8 *)(cs_rows + (wave * 16 + r) * RLD + k * 32 + grp * 8);
        bf16 *dstg = Gf + (int64_t)bcg * (T16 * NJ * 512);
#pragma unroll
        for (int jq = 0; jq < 4; ++jq) {
            const int jt = 4 * bj + jq;
            if (jt * 16 >= Q) break;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k = 0; k < NKN; ++k) {
                const bf16x8 bv = *(const bf16x8 *)(bs_rows + (jq * 16 + r) * RLD + k * 32 + grp * 8);
                acc = mfma_bf16(bv, cf[k], acc);
            }
            // acc[e] = G[i = 16 I + r][j = 16 jt + 4 grp + e]
            const int j0 = jt * 16 + 4 * grp;
            const int J = j0 / 32, q4 = (j0 % 32) / 8, e0 = j0 % 8;
            bf16 o[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = (bf16)acc[e];
            *(u32x2 *)(dstg + (I * NJ + J) * 512 + (r + 16 * q4) * 8 + e0) = *(const u32x2 *)o;
        }
        if (diag) {
            // C fragments of row tile I
            bf16 *dstc = Cf + (int64_t)bcg * (T16 * NKN * 512) + lane * 8;
#pragma unroll
            for (int k = 0; k < NKN; ++k) *(bf16x8 *)(dstc + (I * NKN + k) * 512) = cf[k];
        }
    }
    if (diag) {
        // B^T fragments of 32-blocks J = 2 bi, 2 bi + 1: (t, J) pairs, 2 NTT per block
        bf16 *dstb = Btf + (int64_t)bcg * (N * NJ * 32) + lane * 8;
        for (int f = wave; f < 2 * NTT; f += 4) {
            const int J = 2 * bi + (f & 1), t = f >> 1;
            if (J >= NJ) continue;
            bf16x8 v;
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = bs_rows[((f & 1) * 32 + 8 * grp + e) * RLD + t * 16 + r];
            *(bf16x8 *)(dstb + (t * NJ + J) * 512) = v;
        }
    }
}

// ---------------------------------------------------------------------------
// The single-pass kernel.  256 threads (4 waves); sized for three workgroups
// per CU (51,248 B LDS, <= 168 VGPRs).  Wave w owns state n-tiles {w, w + 4}
// and output tiles {w, 7 - w, 8 + w, 15 - w} (balanced over the triangle).
//   1. loads x, dt and the B^T fragments in one round; decay prefix (wave
//      scans); w_j = exp(cs_last - cs_j)
//   2. x^T staged in LDS (unpadded, chunk-swizzled rows)
//   3. wait for wave w's slice of h_{c-1} (flag of chunk c - 1, or init);
//      issue its loads
//   4. chunk state S_c^T for n-tiles {w, w + 4} (w folded into the B^T
//      fragments); the state slice lands meanwhile
//   5. w replaced by v_j = exp(r_J - cs_j) in LDS; h_c = exp(cs_last) h_{c-1}
//      + S_c to the ring slice (or final_state); h_{c-1} (bf16) to LDS
//   6. output tiles: exp(cs_i) C_i h_{c-1} + intra-chunk product (off-diagonal
//      32-blocks J use exp(cs_i - cs_j) = exp(cs_i - r_J) exp(r_J - cs_j),
//      both factors <= 1, folded into the C B^T fragment; the diagonal
//      32-block takes exp(cs_i - cs_j) [j <= i] element by element) + D x_i,
//      stored as bf16.  The flag is raised after the first tile, once the
//      ring stores have completed.
// ---------------------------------------------------------------------------
// Operands of one 16-row output tile I: its off-diagonal C B^T fragments
// (32-blocks J < I / 2; NG is the most a tile in this slot can have), the
// diagonal one and the four C fragments.  Every slot is loaded (through
// buffer resources over this chunk's blocks: a slot past them reads zero,
// and slots J >= I / 2 go unused), so the number of loads is fixed and none
// sits behind a branch.
template <int NG>
struct TileOps {
    static constexpr int kNG = NG;
    u32x4 g[NG];
    u32x4 gd;
    u32x4 cf[4];
};

template <int NG>
__device__ __forceinline__ void tile_load(TileOps<NG> &t, __amdgpu_buffer_rsrc_t rsG,
                                          __amdgpu_buffer_rsrc_t rsC, int I, int NJ, int lane) {
    const uint32_t gt = (uint32_t)(I * NJ * 512 + lane * 8) * 2u;
    const int Jd = I >> 1;
#pragma unroll
    for (int J = 0; J < NG; ++J) t.g[J] = buf_ld16(rsG, gt + J * 1024u);
    t.gd = buf_ld16(rsG, gt + (uint32_t)Jd * 1024u);
#pragma unroll
    for (int kn = 0; kn < 4; ++kn) t.cf[kn] = buf_ld16(rsC, (uint32_t)(((I * 4 + kn) * 64 + lane) * 8) * 2u);
}

// OPTS: the step is preprocessed (bias, softplus, clamp) and x scaled by the
// step's input factor s_j (Euler or zero-order hold), folded into the
// chunk-state weights, the mask factors v_j and the diagonal mask; the skip
// term keeps the raw x.  s_j takes 1 KB more LDS, so this variant runs two
// workgroups per CU.
template <int P, int N, bool OPTS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 3))) void k_ssd_fused(
    const bf16 *__restrict__ x, const bf16 *__restrict__ dt, const float *__restrict__ A,
    const bf16 *__restrict__ Btf, const bf16 *__restrict__ Cf, const bf16 *__restrict__ Gf,
    const float *__restrict__ D, const float *init, bf16 *__restrict__ y, float *fin,
    float *ring, int *flags, int L, int H, int G, int Q, int nc, int nbh, DtOpts o) {
    constexpr int PT = P / 16, NT = N / 16, NTW = NT / 4, NKN = N / 32;
    static_assert(NT % 4 == 0 && N % 32 == 0, "N must be a multiple of 64");
    constexpr int XW = 256, HW = N;   // unpadded rows, chunk-swizzled (swz)
    __shared__ float cs_s[256];
    __shared__ float s_s[OPTS ? 256 : 1];  // input factor of each step (OPTS)
    // w_j = exp(cs_last - cs_j) (chunk-state weights) until step 4 is done in
    // every wave, then v_j = exp(r_J(j) - cs_j) (intra-chunk mask factor).
    // One array keeps the workgroup within a third of the CU's LDS.
    __shared__ float wv_s[256];
    __shared__ float wsum_s[4];
    __shared__ float ref_s[8];   // r_J: cs at the last step of 32-block J
    __shared__ bf16 xs[P * XW];
    __shared__ bf16 hs[P * HW];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar offsets
    const int r = lane & 15, grp = lane >> 4;
    // Work item.  Workgroups are dealt round-robin to 8 streams (block k ->
    // stream k % 8, the XCD round-robin); stream x walks chunk-columns
    // c = 0, 1, ... over its own eighth of the (b, h) pairs, so the
    // predecessor (c - 1, b, h) of every item is block k - nbh: same stream,
    // smaller id.  With in-order dispatch inside a stream, the lowest
    // unfinished block is always resident and its predecessor is done, so
    // the chain drains; the bounded wait below is a backstop.
    int c, bh;
    {
        const int k = blockIdx.x;
        if (nbh % 8 == 0) {
            const int per = nbh / 8, m = k >> 3;
            c = m / per;
            bh = (k & 7) * per + (m - c * per);
        } else {
            c = k / nbh;
            bh = k - c * nbh;
        }
    }
    const int b = bh / H;
    const int h = bh - b * H;
    const int g = h / (H / G);
    const int s = c * Q;
    const int q = min(Q, L - s);
    const int nb = (q + 31) / 32;          // 32-step blocks holding data
    const int T16 = (q + 15) / 16;
    const int NJ = (Q + 31) / 32, T16Q = Q / 16;
    const u32x4 z4 = {0u, 0u, 0u, 0u};
    const int bcg = (b * nc + c) * G + g;
    const bf16 *Btc = Btf + bcg * (N * NJ * 32);
    const bf16 *Gfc = Gf + bcg * (T16Q * NJ * 512);
    const bf16 *Cfc = Cf + bcg * (T16Q * NKN * 512);
    constexpr int PN = P * N;

    // dt, x and B^T in one round, dt first (the decay prefix waits for it
    // alone).  Every load goes through a buffer resource, a lane with nothing
    // to load pointing past its end, so none sits behind a branch and the
    // compiler's counted waits leave the later loads in flight.
    const int row0 = (b * L + s) * H + h;
    const auto rsY = buf_rsrc(y + row0 * P, (uint32_t)q * H * P * 2u);
    const auto rsDt = buf_rsrc(dt + (b * L + s) * H + h, (uint32_t)q * H * 2u);
    const uint16_t dt_raw = buf_ld2(rsDt, tid < q ? (uint32_t)tid * H * 2u : kBufOff);
    XStage<P> xst;
    stage_x_load<P>(xst, x + row0 * P, H * P, q);
    // B^T fragments (rows past q are stored as zero; blocks past NJ read as zero, unused)
    const auto rsBt = buf_rsrc(Btc, (uint32_t)(N * NJ * 32) * 2u);
    bf16x8 bfr[8][NTW];
#pragma unroll
    for (int J = 0; J < 8; ++J)
#pragma unroll
        for (int tt = 0; tt < NTW; ++tt)
            bfr[J][tt] = as_bf16x8(buf_ld16(
                rsBt, J < NJ ? (uint32_t)((((wave + 4 * tt) * NJ + J) * 64 + lane) * 8) * 2u : kBufOff));
    // keep the whole round here: the scheduler would otherwise sink B^T loads
    // towards their use, behind the ring loads that must land during step 4
    __builtin_amdgcn_sched_barrier(0);

    // 1. decay prefix
    float sx_own = 1.f;  // this thread's step's input factor (OPTS)
    {
        float v;
        if constexpr (OPTS) {
            const float de = (tid < q) ? dt_effective((float)__builtin_bit_cast(bf16, dt_raw), h, o) : 0.f;
            sx_own = (tid < q) ? input_scale(de, A[h], o.scale) : 0.f;
            s_s[tid] = sx_own;
            v = de * A[h];
        } else {
            v = (tid < q) ? (float)__builtin_bit_cast(bf16, dt_raw) * A[h] : 0.f;
        }
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float o = __shfl_up(v, off, 64);
            if (lane >= off) v += o;
        }
        // (LDS-only barriers: the x and B^T loads stay in flight)
        if (lane == 63) wsum_s[wave] = v;
        lds_barrier();
        for (int w = 0; w < wave; ++w) v += wsum_s[w];
        cs_s[tid] = v;  // past q: repeats the last valid value
        lds_barrier();
        if (tid < 8) ref_s[tid] = cs_s[min(32 * tid + 31, q - 1)];
        wv_s[tid] = __expf(cs_s[q - 1] - v) * sx_own;
    }
    const float cs_last = cs_s[q - 1];

    // 2. stage x^T (rows past q were loaded as zero)
    stage_x_write_swz<P>(xst, xs);
    lds_barrier();

    // 3. hand-off, first half: wait until wave `wave` of chunk c - 1 of this
    // (b, h) has published its slice of h_{c-1}, then load the slice (it
    // arrives while the chunk state is computed).  The ring is read and
    // written with agent-coherent accesses (see ld_agent_f32x4), in a
    // lane-major layout so each wave moves one contiguous 1 KiB block per
    // access; init / final_state use the [P][N] layout.
    // hv[tt][pt][e] = h_{c-1}[p = 16 pt + r][n = 16 (wave + 4 tt) + 4 grp + e]
    // sits at float ring_base(tt) + 256 pt of the (b, h) slice; the per-pt
    // part folds into the access's immediate offset
    auto ring_base = [&](int tt) -> int { return ((wave * NTW + tt) * PT * 64 + lane) * 4; };
    int *myflag = flags + bh * 4 + wave;
    const bool have_h = c > 0 || init != nullptr;
    f32x4 hv[NTW][PT];
    // The first round (B^T above all) has landed by now; waiting for it here
    // leaves only this hand-off's loads in flight on either branch, so the
    // chunk-state MFMAs below need no wait (after the join the compiler
    // would otherwise wait for most of the ring loads).
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    if (c > 0) {
        int n = 0;
        while (__hip_atomic_load(myflag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < c && n < kSpinLimit) {
            __builtin_amdgcn_s_sleep(1);
            ++n;
        }
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        const auto rsH = buf_rsrc(ring + ((c - 1) & 1) * nbh * PN + bh * PN, (uint32_t)PN * 4u);
#pragma unroll
        for (int tt = 0; tt < NTW; ++tt)
#pragma unroll
            for (int pt = 0; pt < PT; ++pt)
                hv[tt][pt] = ld_agent_f32x4(rsH, (uint32_t)(ring_base(tt) + pt * 256) * 4u);
    } else {
#pragma unroll
        for (int tt = 0; tt < NTW; ++tt)
#pragma unroll
            for (int pt = 0; pt < PT; ++pt)
                hv[tt][pt] = init ? *(const f32x4 *)(init + bh * PN + (pt * 16 + r) * N + (wave + 4 * tt) * 16 + 4 * grp)
                                  : f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // 4. chunk state: acc_s[tt][pt] = S^T[n = 16 (wave + 4 tt) + 4 grp + e][p = 16 pt + r]
    f32x4 acc_s[NTW][PT];
#pragma unroll
    for (int tt = 0; tt < NTW; ++tt)
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) acc_s[tt][pt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int J = 0; J < 8; ++J) {
        if (J < nb) {
            const f32x4 w0 = *(const f32x4 *)(wv_s + 32 * J + grp * 8);
            const f32x4 w1 = *(const f32x4 *)(wv_s + 32 * J + grp * 8 + 4);
            bf16x8 bx[PT];
#pragma unroll
            for (int pt = 0; pt < PT; ++pt)
                bx[pt] = *(const bf16x8 *)(xs + swz<XW>(pt * 16 + r, 32 * J + grp * 8));
#pragma unroll
            for (int tt = 0; tt < NTW; ++tt) {
                bf16x8 a = bfr[J][tt];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    a[e] = (bf16)((float)a[e] * w0[e]);
                    a[e + 4] = (bf16)((float)a[e + 4] * w1[e]);
                }
#pragma unroll
                for (int pt = 0; pt < PT; ++pt) acc_s[tt][pt] = mfma_bf16(a, bx[pt], acc_s[tt][pt]);
            }
        }
    }

    // Output tiles of this wave: T_k = {w, 7 - w, 8 + w, 15 - w}; tile T_k has
    // at most 2k + 1 off-diagonal 32-blocks.  Tile 0's operands load now (they
    // land during the hand-off), tiles 1 and 2 after it, tile 3 after tile 0.
    // With every tile of a full chunk valid, each load count is fixed, so the
    // wait before raising the flag can leave the later tiles' loads in flight.
    const int tI[4] = {wave, 7 - wave, 8 + wave, 15 - wave};
    const auto rsG = buf_rsrc(Gfc, (uint32_t)(T16Q * NJ * 512) * 2u);
    const auto rsC = buf_rsrc(Cfc, (uint32_t)(T16Q * NKN * 512) * 2u);
    TileOps<1> t0;
    TileOps<3> t1;
    TileOps<5> t2;
    TileOps<7> t3;
    tile_load(t0, rsG, rsC, tI[0], NJ, lane);

    lds_barrier();  // step 4 is done in every wave: w may be replaced by v
    // v_j relative to the end of j's own 32-block (cs past q repeats)
    wv_s[tid] = __expf(ref_s[tid >> 5] - cs_s[tid]) * sx_own;

    // 5. hand-off, second half: h_c = exp(cs_last) h_{c-1} + S_c to this
    // wave's ring slice (or final_state); h_{c-1} as bf16 to LDS.  The wave
    // raises its flag after its first output tile, once these stores have
    // completed.
    const float lam_c = __expf(cs_last);
    const bool last = c == nc - 1;
    float *hout = last ? (fin ? fin + bh * PN : nullptr) : ring + (c & 1) * nbh * PN + bh * PN;
    const auto rsO = buf_rsrc(hout, (uint32_t)PN * 4u);
    // Tile 0's loads (issued before the barrier above, long landed) are waited
    // for here, before the ring stores: with loads and stores both in flight
    // the compiler's wait for them would also wait for most of the stores.
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
#pragma unroll
    for (int tt = 0; tt < NTW; ++tt) {
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) {
            const int p = pt * 16 + r, n0 = (wave + 4 * tt) * 16 + 4 * grp;
            const f32x4 hn = lam_c * hv[tt][pt] + acc_s[tt][pt];
            if (hout) {
                if (last) {
                    *(f32x4 *)(hout + p * N + n0) = hn;
                } else {
                    st_agent_f32x4(hn, rsO, (uint32_t)(ring_base(tt) + pt * 256) * 4u);
                }
            }
            bf16 hb[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) hb[e] = (bf16)hv[tt][pt][e];
            *(u32x2 *)(hs + swz<HW>(p, n0)) = *(const u32x2 *)hb;
        }
    }
    lds_barrier();  // hs and v complete in every wave

    // 6. output tiles
    const float Dh = D ? D[h] : 0.f;
    tile_load(t1, rsG, rsC, tI[1], NJ, lane);
    tile_load(t2, rsG, rsC, tI[2], NJ, lane);

    // acc[pt][e] = y[i = 16 I + r][p = 16 pt + 4 grp + e] (D[m = p][n = i] of the MFMAs):
    // the state term exp(cs_i) C_i h_{c-1} first (scaled once), then the intra product
    auto compute_tile = [&](const auto &t, int I, f32x4(&acc)[PT]) {
        constexpr int NG = std::decay_t<decltype(t)>::kNG;
        const int il = I * 16 + r;
        const float csi = cs_s[il];
        const int Jd = I >> 1;
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) acc[pt] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (have_h) {
#pragma unroll
            for (int kn = 0; kn < NKN; ++kn) {
#pragma unroll
                for (int pt = 0; pt < PT; ++pt) {
                    const bf16x8 ah = *(const bf16x8 *)(hs + swz<HW>(pt * 16 + r, kn * 32 + grp * 8));
                    acc[pt] = mfma_bf16(ah, as_bf16x8(t.cf[kn]), acc[pt]);
                }
            }
            const float ei = __expf(csi);
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) acc[pt] *= ei;
        }
#pragma unroll
        for (int J = 0; J < NG; ++J) {
            if (J < Jd) {
                const float u = __expf(csi - ref_s[J]);
                const f32x4 v0 = *(const f32x4 *)(wv_s + 32 * J + grp * 8);
                const f32x4 v1 = *(const f32x4 *)(wv_s + 32 * J + grp * 8 + 4);
                bf16x8 gm = as_bf16x8(t.g[J]);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    gm[e] = (bf16)((float)gm[e] * (u * v0[e]));
                    gm[e + 4] = (bf16)((float)gm[e + 4] * (u * v1[e]));
                }
#pragma unroll
                for (int pt = 0; pt < PT; ++pt) {
                    const bf16x8 ax = *(const bf16x8 *)(xs + swz<XW>(pt * 16 + r, 32 * J + grp * 8));
                    acc[pt] = mfma_bf16(ax, gm, acc[pt]);
                }
            }
        }
        const int jl = 32 * Jd + grp * 8;
        const bf16x8 gd = as_bf16x8(t.gd);
        bf16x8 bm;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int j = jl + e;
            const float sj = OPTS ? s_s[j] : 1.f;
            bm[e] = (bf16)((j <= il) ? __expf(csi - cs_s[j]) * (float)gd[e] * sj : 0.f);
        }
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) {
            const bf16x8 ax = *(const bf16x8 *)(xs + swz<XW>(pt * 16 + r, jl));
            acc[pt] = mfma_bf16(ax, bm, acc[pt]);
        }
    };
    // + D x_i, to bf16.  Lane (r, grp) holds row i = 16 I + r, columns 16 pt +
    // 4 grp .. + 3 (block M[grp][pt]).  A butterfly over lane ^ 16, lane ^ 32
    // transposes the 4 x 4 block grid so lane group g holds M[0..3][g] =
    // columns 16 g .. 16 g + 15: two 16-byte stores per lane.
    auto store_tile = [&](int I, const f32x4(&acc)[PT]) {
        const int il = I * 16 + r;
        // x[i][16 pt + 4 grp + e] = xs[swz(16 pt + 4 grp + e, il)]; row & 15 = 4 grp + e,
        // so the swizzled column offset depends on e only
        int xoff[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) xoff[e] = (4 * grp + e) * XW + swz<XW>(4 * grp + e, il) - (4 * grp + e) * XW;
        u32x2 m[PT];
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) {
            bf16 o[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = (bf16)(acc[pt][e] + Dh * (float)xs[pt * 16 * XW + xoff[e]]);
            m[pt] = *(const u32x2 *)o;
        }
        auto xchg = [](u32x2 v, int mask) {
            return u32x2{(uint32_t)__shfl_xor((int)v[0], mask, 64), (uint32_t)__shfl_xor((int)v[1], mask, 64)};
        };
        const bool g1 = grp & 1, g2 = grp & 2;
        // stage 1: keep the columns of this lane's parity, swap the rest with g ^ 1
        const u32x2 c0 = g1 ? m[1] : m[0], c2 = g1 ? m[3] : m[2];                      // M[g][g&1], M[g][2+(g&1)]
        const u32x2 c1 = xchg(g1 ? m[0] : m[1], 16), c3 = xchg(g1 ? m[2] : m[3], 16);  // M[g^1][..]
        // stage 2: keep column g, swap column g ^ 2 with g ^ 2
        const u32x2 t0v = g2 ? c2 : c0, t1v = g2 ? c3 : c1;                              // M[g][g], M[g^1][g]
        const u32x2 t2v = xchg(g2 ? c0 : c2, 32), t3v = xchg(g2 ? c1 : c3, 32);          // M[g^2][g], M[g^3][g]
        // order by source row: out[s] = t[s ^ g]
        const u32x2 a0 = g1 ? t1v : t0v, a1 = g1 ? t0v : t1v, a2 = g1 ? t3v : t2v, a3 = g1 ? t2v : t3v;
        const u32x2 o0 = g2 ? a2 : a0, o1 = g2 ? a3 : a1, o2 = g2 ? a0 : a2, o3 = g2 ? a1 : a3;
        // rows past q: offsets past the resource's end (no branch around the stores)
        const uint32_t yo = il < q ? (uint32_t)(il * H * P + 16 * grp) * 2u : kBufOff;
        buf_st16(u32x4{o0[0], o0[1], o1[0], o1[1]}, rsY, yo);
        buf_st16(u32x4{o2[0], o2[1], o3[0], o3[1]}, rsY, yo + 16u);
    };

    // Every tile is computed and stored without a branch (a tile past q, in a
    // short last chunk, computes on zero operands and its stores are dropped),
    // so the compiler's counted waits keep tile 3's loads in flight.
    f32x4 acc[PT];
    compute_tile(t0, tI[0], acc);
    if (!last) {
        // this wave's ring slice is complete: raise its flag (the loads of
        // tiles 1 and 2, issued above, are waited for here too)
        __builtin_amdgcn_s_waitcnt(0);
        if (lane == 0) __hip_atomic_store(myflag, c + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    store_tile(tI[0], acc);
    tile_load(t3, rsG, rsC, tI[3], NJ, lane);
    compute_tile(t1, tI[1], acc);
    store_tile(tI[1], acc);
    compute_tile(t2, tI[2], acc);
    store_tile(tI[2], acc);
    compute_tile(t3, tI[3], acc);
    store_tile(tI[3], acc);
}

bool fused_supported(const Dims &d) {
    if (!(d.dtype == 1 && d.P == 64 && d.N == 128 && d.Q <= 256 && d.nc >= 1)) return false;
    // element offsets inside the single-pass kernel are 32-bit
    const int64_t lim = (int64_t)1 << 31;
    const int64_t nbh = d.b * d.H, T16 = d.Q / 16, NJ = (d.Q + 31) / 32, nbcg = d.b * d.nc * d.G;
    return d.b * d.L * d.H * d.P < lim && d.nc * nbh < lim && 2 * nbh * d.P * d.N < lim &&
           nbcg * T16 * NJ * 512 < lim && nbcg * d.N * NJ * 32 < lim && nbcg * T16 * (d.N / 32) * 512 < lim;
}

hipError_t launch_fused_prep(const Dims &d, const void *B, const void *C, void *Gf, void *Btf,
                             void *Cf, int *flags, hipStream_t st) {
    const int T64 = (int)((d.Q + 63) / 64);
    dim3 grid((unsigned)(d.b * d.nc * d.G), (unsigned)(T64 * (T64 + 1) / 2));
    k_fused_prep<128><<<grid, 256, 0, st>>>((const bf16 *)B, (const bf16 *)C, (bf16 *)Gf, (bf16 *)Btf,
                                            (bf16 *)Cf, flags, (int)(d.b * d.H * 4), (int)d.L, (int)d.G,
                                            (int)d.Q, (int)d.nc);
    return hipGetLastError();
}

hipError_t launch_fused_main(const Dims &d, const void *x, const void *dt, const float *A,
                             const void *Btf, const void *Cf, const void *Gf, const float *D,
                             const float *init, void *y, float *fin, float *ring, int *flags,
                             hipStream_t st, const DtOpts *o) {
    const unsigned grid = (unsigned)(d.b * d.nc * d.H);
    if (o)
        k_ssd_fused<64, 128, true><<<grid, 256, 0, st>>>(
            (const bf16 *)x, (const bf16 *)dt, A, (const bf16 *)Btf, (const bf16 *)Cf, (const bf16 *)Gf,
            D, init, (bf16 *)y, fin, ring, flags, (int)d.L, (int)d.H, (int)d.G, (int)d.Q, (int)d.nc,
            (int)(d.b * d.H), *o);
    else
        k_ssd_fused<64, 128, false><<<grid, 256, 0, st>>>(
            (const bf16 *)x, (const bf16 *)dt, A, (const bf16 *)Btf, (const bf16 *)Cf, (const bf16 *)Gf,
            D, init, (bf16 *)y, fin, ring, flags, (int)d.L, (int)d.H, (int)d.G, (int)d.Q, (int)d.nc,
            (int)(d.b * d.H), DtOpts{nullptr, 0.f, 0.f, 0, 0});
    return hipGetLastError();
}

}  // namespace ssd
