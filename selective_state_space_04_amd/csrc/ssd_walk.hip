// Single-pass SSD forward for bfloat16 inputs (gfx950): one workgroup walks
// one (b, h) sequence from start to end and keeps its state on chip.
//
// The chunked algorithm (Mamba-2 review, docsaid.org, section
// "2つのルートを半分ずつ"; SSD summary, section "チャンク化アルゴリズム") with
// 32-step chunks: inside a chunk the masked attention form, across chunks only
// the chunk-end state, which here never leaves the MFMA accumulators.  Every
// (b, h) pair is independent, so the walk needs no hand-off between
// workgroups; x is read once and y written once, and the only other traffic
// is the per-chunk operands shared by all heads of a group (read from L2).
//
// Per chunk of 32 steps starting at state h (P x N, held transposed as
// h[n][p] in fp32 accumulators), with c_j = sum of dt A over the chunk's
// steps up to and including j (so exp(c_i - c_j) = a_{j+1} ... a_i, the mask
// of the review's section "A を一つの数に簡略化する"):
//   y_i   = exp(c_i) C_i h + sum_{j<=i} exp(c_i - c_j) (C_i . B_j) s_j x_j + D x_i
//   h_end = exp(c_last) h + sum_j exp(c_last - c_j) s_j B_j x_j^T
// (s_j = 1 unless an input scale is requested).  The decay is carried as a
// running log2 scale Ls: the accumulators hold g = h / 2^Ls, and with
// E_j = 2^-(Ls + c_j) s_j x_j
//   y_i  = 2^(Ls + c_i) [C_i g + sum_{j<=i} (C_i . B_j) E_j] + D x_i
//   g'   = g + B^T E,   Ls' = Ls + c_last,
// so the causal C B^T tile of the chunk is the same for every head (it is
// precomputed once per group) and the per-head work is one factor per step.
// The factors stay within 2^+-64: a chunk that would leave that range takes a
// path with the per-element factors exp(c_i - c_j) <= 1, exp(c_last - c_j)
// <= 1, which also folds 2^Ls back into the accumulators (Ls restarts at 0).
//
// Operand layouts (MFMA v_mfma_f32_16x16x32_bf16, lane l: r = l % 16,
// gq = l / 16).  The 32 steps of a chunk are the contraction index of the
// diagonal and state-update products; lane group gq holds the steps
// kset(gq) = {4 gq .. 4 gq + 3, 16 + 4 gq .. 16 + 4 gq + 3}, which are the
// rows an accumulator tile gives lane group gq, so the state accumulators
// convert to bf16 operands in place.  The state contraction over n uses the
// same grouping of n within each 32-wide step s.
#include "ssd_device.h"
#include "ssd_launch.h"

namespace ssd {

namespace {

constexpr int kBlk = 32;                 // steps per chunk
constexpr int kOpsBytes = 18432;         // C (8 KiB), B^T (8 KiB), causal C B^T (2 KiB) fragments
constexpr int kOffBt = 8192, kOffG = 16384;
constexpr float kRange = 64.f;           // |log2| bound on every factor of the fast path

template <bool OPTS> struct Rec {
    // per (b, chunk, h): c_0 .. c_31 (log2 units), c_last, cmin, cmax, 0
    // [, s_0 .. s_31 (input scale)]
    static constexpr int kFloats = OPTS ? 68 : 36;
    static constexpr int kPieces = kFloats / 4;
};

// 16-byte chunk `chunk` (0..7) of x-tile row `row` is stored at this chunk
// position: the 32-byte pair index is XORed with bits 1..2 of the row, so the
// rows a transposing read or a row read touches (r0 + 0..15) fall on every
// 32-byte bank window of a 256-byte span twice.
__device__ __forceinline__ int xt_pos(int row, int chunk) {
    return ((((chunk >> 1) ^ (row >> 1)) & 3) << 1) | (chunk & 1);
}

// s_waitcnt for vmcnt <= N only (expcnt and lgkmcnt left at their maxima).
template <int N> __device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

__device__ __forceinline__ float exp2_raw(float v) { return __builtin_amdgcn_exp2f(v); }

__device__ __forceinline__ float rfl(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, v)));
}

// MFMA fragment of column c0 + r of the x tile, steps kset(gq): two transposing
// reads, of rows 4 gq .. 4 gq + 3 and 16 + 4 gq .. 16 + 4 gq + 3.
__device__ __forceinline__ bf16x8 x_frag(const unsigned char *xt, int c0, int lane) {
    const int j = lane & 15, gq = lane >> 4;
    const int col = c0 + 4 * (j & 3);
    const int ch = col >> 3, half = (col >> 2) & 1;
    const int row0 = 4 * gq + (j >> 2), row1 = row0 + 16;
    const unsigned char *a0 = xt + row0 * 128 + xt_pos(row0, ch) * 16 + half * 8;
    const unsigned char *a1 = xt + row1 * 128 + xt_pos(row1, ch) * 16 + half * 8;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4 *)a0);
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4 *)a1);
    bf16x8 f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const short a = lo[e], b = hi[e];
        f[e] = __builtin_bit_cast(bf16, a);
        f[e + 4] = __builtin_bit_cast(bf16, b);
    }
    return f;
}

// Four consecutive x values (col % 4 == 0) of tile row `row`.
__device__ __forceinline__ u32x2 x_row4(const unsigned char *xt, int row, int col) {
    return *(const u32x2 *)(xt + row * 128 + xt_pos(row, col >> 3) * 16 + ((col >> 2) & 1) * 8);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    const bf16x2 v = {(bf16)a, (bf16)b};  // one v_cvt_pk_bf16_f32
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __builtin_bit_cast(float, v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __builtin_bit_cast(float, v & 0xffff0000u); }

// Copies from global memory straight into LDS (global_load_lds_dwordx4): copy
// m moves 16 bytes per lane from sbase + voff + 1024 m to LDS
// lds + 1024 m + 16 lane (the immediate offset applies to both addresses).
// Written as inline assembly so the compiler does not see the LDS writes: it
// would otherwise wait for every copy in flight before each LDS read.  The
// callers wait for the copies themselves (vmcnt) before reading what they
// wrote.  One wait state separates the M0 write from the copy that reads it.
template <int NC>
__device__ __forceinline__ void dma16(uint32_t voff, const void *sbase, uint32_t lds) {
    static_assert(NC >= 1 && NC <= 4, "one to four copies");
    if constexpr (NC == 4)
        asm volatile(
            "s_mov_b32 m0, %2\n\ts_nop 0\n\t"
            "global_load_lds_dwordx4 %0, %1\n\t"
            "global_load_lds_dwordx4 %0, %1 offset:1024\n\t"
            "global_load_lds_dwordx4 %0, %1 offset:2048\n\t"
            "global_load_lds_dwordx4 %0, %1 offset:3072"
            :
            : "v"(voff), "s"(sbase), "s"(lds)
            : "memory", "m0");
    else if constexpr (NC == 3)
        asm volatile(
            "s_mov_b32 m0, %2\n\ts_nop 0\n\t"
            "global_load_lds_dwordx4 %0, %1\n\t"
            "global_load_lds_dwordx4 %0, %1 offset:1024\n\t"
            "global_load_lds_dwordx4 %0, %1 offset:2048"
            :
            : "v"(voff), "s"(sbase), "s"(lds)
            : "memory", "m0");
    else if constexpr (NC == 2)
        asm volatile(
            "s_mov_b32 m0, %2\n\ts_nop 0\n\t"
            "global_load_lds_dwordx4 %0, %1\n\t"
            "global_load_lds_dwordx4 %0, %1 offset:1024"
            :
            : "v"(voff), "s"(sbase), "s"(lds)
            : "memory", "m0");
    else
        asm volatile(
            "s_mov_b32 m0, %2\n\ts_nop 0\n\t"
            "global_load_lds_dwordx4 %0, %1"
            :
            : "v"(voff), "s"(sbase), "s"(lds)
            : "memory", "m0");
}

// Four copies with one per-lane offset each (the x tile): copy m reads
// sbase + v[m] + 1024 m and writes LDS lds + 1024 m + 16 lane.
__device__ __forceinline__ void dma16_4v(uint32_t v0, uint32_t v1, uint32_t v2, uint32_t v3, const void *sbase,
                                         uint32_t lds) {
    asm volatile(
        "s_mov_b32 m0, %5\n\ts_nop 0\n\t"
        "global_load_lds_dwordx4 %0, %4\n\t"
        "global_load_lds_dwordx4 %1, %4 offset:1024\n\t"
        "global_load_lds_dwordx4 %2, %4 offset:2048\n\t"
        "global_load_lds_dwordx4 %3, %4 offset:3072"
        :
        : "v"(v0), "v"(v1), "v"(v2), "v"(v3), "s"(sbase), "s"(lds)
        : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}

// Copy instructions of one chunk (1 KiB of the slot each): 0 .. 17 the
// group's operand fragments, 18 .. 21 the x tile, 22 the decay record (lanes
// past the record repeat its last piece into the slot's padding).
constexpr int kInsOps = kOpsBytes / 1024, kInsX = 4, kInsAll = kInsOps + kInsX + 1;

// Per-lane byte offsets of the x-tile copies m = 0..3 (tile rows 8 m + lane /
// 8, clamped to rowlim), relative to a base kXBias bytes below the tile's
// first row: copy m's immediate adds 1024 m, so its offset is the row offset
// plus kXBias - 1024 m, never negative (the offset register is unsigned).
constexpr int kXBias = 1024 * (kInsX - 1);
struct XOffsets {
    uint32_t v[kInsX];
};

__device__ __forceinline__ XOffsets x_offsets(int lane, int rowlim, int H) {
    XOffsets o;
#pragma unroll
    for (int m = 0; m < kInsX; ++m) {
        const int row = 8 * m + (lane >> 3);
        o.v[m] = (uint32_t)((min(row, rowlim) * H * 64 + xt_pos(row, lane & 7) * 8) * 2) + (uint32_t)(kXBias - 1024 * m);
    }
    return o;
}

}  // namespace

// ---------------------------------------------------------------------------
// Preparation: for every chunk (b, k) of 32 steps
//   ops[b][k][g] (18 KiB, one per group) in MFMA-fragment order, lane l at
//   byte 16 l of each 1 KiB fragment:
//     C   frag (rt, s): C[16 rt + r][32 s + 4 gq .. + 3], C[16 rt + r][32 s + 16 + 4 gq .. + 3]
//     B^T frag nt:      B[j][16 nt + r] for j in kset(gq)
//     CB  frag rt:      (C_i . B_j) [j <= i], i = 16 rt + r, j in kset(gq)
//   rec[b][k][h]: the decay prefix c_j = sum_{t0 <= t <= t0 + j} dt_t A_h log2(e)
//     (steps past L add nothing), c_last, its min and max over the chunk,
//     and with options the input scale s_j of each step.
// Rows past L are zero.  blockIdx.y < G: the operands of group blockIdx.y;
// blockIdx.y == G: the decay records of every head.
// ---------------------------------------------------------------------------
template <bool OPTS>
__global__ __launch_bounds__(256) void k_walk_prep(const bf16 *__restrict__ B, const bf16 *__restrict__ C,
                                                   const bf16 *__restrict__ dt, const float *__restrict__ A,
                                                   unsigned char *__restrict__ ops, float *__restrict__ rec,
                                                   int L, int H, int G, int nblk, DtOpts o) {
    constexpr int N = 128, RLD = N + 8;
    const int bk = blockIdx.x;
    const int k = bk % nblk, b = bk / nblk;
    const int t0 = k * kBlk, q = min(kBlk, L - t0);
    const int tid = threadIdx.x;

    if ((int)blockIdx.y == G) {
        constexpr int RF = Rec<OPTS>::kFloats;
        const float l2e = 1.4426950408889634f;
        for (int h = tid; h < H; h += 256) {
            const float Ah = A[h], a2 = Ah * l2e;
            // every load issued before the first use (rows past L clamped and
            // then given no weight), so they are all in flight together
            const bf16 *src = dt + ((int64_t)b * L + t0) * H + h;
            bf16 raw[kBlk];
#pragma unroll
            for (int j = 0; j < kBlk; ++j) raw[j] = src[(int64_t)min(j, q - 1) * H];
            float cv[kBlk], sv[kBlk];
            float c = 0.f, cmin = 0.f, cmax = 0.f;
#pragma unroll
            for (int j = 0; j < kBlk; ++j) {
                float d = (float)raw[j], sj = 1.f;
                if constexpr (OPTS) {
                    d = dt_effective(d, h, o);
                    sj = input_scale(d, Ah, o.scale);
                }
                const float dA = j < q ? d * a2 : 0.f;
                c += dA;
                cv[j] = c;
                sv[j] = j < q ? sj : 0.f;
                cmin = fminf(cmin, c);
                cmax = fmaxf(cmax, c);
            }
            float *dst = rec + ((int64_t)bk * H + h) * RF;
#pragma unroll
            for (int j = 0; j < kBlk; j += 4) *(f32x4 *)(dst + j) = f32x4{cv[j], cv[j + 1], cv[j + 2], cv[j + 3]};
            *(f32x4 *)(dst + 32) = f32x4{c, cmin, cmax, 0.f};
            if constexpr (OPTS) {
#pragma unroll
                for (int j = 0; j < kBlk; j += 4)
                    *(f32x4 *)(dst + 36 + j) = f32x4{sv[j], sv[j + 1], sv[j + 2], sv[j + 3]};
            }
        }
        return;
    }

    const int g = blockIdx.y;
    __shared__ bf16 cs_[kBlk * RLD];
    __shared__ bf16 bs_[kBlk * RLD];
    const int lane = tid & 63, wave = tid >> 6;
    const int r = lane & 15, gq = lane >> 4;
    const u32x4 z = {0u, 0u, 0u, 0u};
    const int64_t ld = (int64_t)G * N;
    const bf16 *Cb = C + ((int64_t)b * L + t0) * ld + (int64_t)g * N;
    const bf16 *Bb = B + ((int64_t)b * L + t0) * ld + (int64_t)g * N;
    for (int it = tid; it < kBlk * (N / 8); it += 256) {
        const int row = it / (N / 8), ch = it % (N / 8);
        const int rr = min(row, q - 1);
        const u32x4 vc = *(const u32x4 *)(Cb + rr * ld + ch * 8);
        const u32x4 vb = *(const u32x4 *)(Bb + rr * ld + ch * 8);
        *(u32x4 *)(cs_ + row * RLD + ch * 8) = row < q ? vc : z;
        *(u32x4 *)(bs_ + row * RLD + ch * 8) = row < q ? vb : z;
    }
    __syncthreads();
    unsigned char *dst = ops + ((int64_t)bk * G + g) * kOpsBytes;
    for (int it = tid; it < 8 * 64; it += 256) {
        const int f = it >> 6, l = it & 63, rr = l & 15, gg = l >> 4;
        // C fragment (rt, s) = (f / 4, f % 4)
        {
            const int rt = f >> 2, s = f & 3;
            const bf16 *row = cs_ + (16 * rt + rr) * RLD + 32 * s + 4 * gg;
            const u32x2 lo = *(const u32x2 *)row, hi = *(const u32x2 *)(row + 16);
            *(u32x4 *)(dst + f * 1024 + 16 * l) = u32x4{lo[0], lo[1], hi[0], hi[1]};
        }
        // B^T fragment nt = f
        {
            bf16x8 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                v[e] = bs_[(4 * gg + e) * RLD + 16 * f + rr];
                v[e + 4] = bs_[(16 + 4 * gg + e) * RLD + 16 * f + rr];
            }
            *(bf16x8 *)(dst + kOffBt + f * 1024 + 16 * l) = v;
        }
    }
    if (wave < 2) {
        // causal C B^T rows 16 rt .. 16 rt + 15: D[m = j][n = i] = B_j . C_i
        const int rt = wave;
        f32x4 d0 = {0.f, 0.f, 0.f, 0.f}, d1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < N / 32; ++s) {
            const bf16x8 cf = *(const bf16x8 *)(cs_ + (16 * rt + r) * RLD + 32 * s + 8 * gq);
            const bf16x8 b0 = *(const bf16x8 *)(bs_ + r * RLD + 32 * s + 8 * gq);
            const bf16x8 b1 = *(const bf16x8 *)(bs_ + (16 + r) * RLD + 32 * s + 8 * gq);
            d0 = mfma_bf16(b0, cf, d0);
            d1 = mfma_bf16(b1, cf, d1);
        }
        // lane (r, gq): d0[e] = C_i . B_j for i = 16 rt + r, j = 4 gq + e; d1: j = 16 + 4 gq + e
        const int i = 16 * rt + r;
        bf16x8 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            v[e] = (bf16)(4 * gq + e <= i ? d0[e] : 0.f);
            v[e + 4] = (bf16)(16 + 4 * gq + e <= i ? d1[e] : 0.f);
        }
        *(bf16x8 *)(dst + kOffG + rt * 1024 + 16 * lane) = v;
    }
}

// ---------------------------------------------------------------------------
// The walk.  Workgroup = NH heads of one batch (same group) and 2 NH + 1
// waves: compute wave 2 hh + w owns columns 32 w .. 32 w + 31 of head h0 + hh
// (two 16-column MFMA tiles), and the last wave only moves data.  That copy
// wave streams each chunk's operands (its group's fragments), the heads' x
// tiles and decay records straight into LDS rings (dma16) several chunks
// ahead, waits for them itself (vector memory operations retire in issue
// order), and turns each record into the factors the compute waves use
// (below); one barrier per chunk hands a chunk over.  The compute waves
// touch global memory only to store y, so they never wait on a copy, and
// they overlap the state products of chunk k with the output of chunk k - 1
// and the scaled x of chunk k + 1.
//
// Factors of chunk m and head hh (LDS, written two chunks ahead, in the
// copy wave's per-head running scale Ls):
//   fast chunk:  F0_j = 2^-(Ls + c_j) s_j, F1_i = 2^(Ls + c_i), then Ls += c_last;
//     a chunk out of range with Ls but in range on its own first folds 2^Ls
//     into the state (resc) and restarts Ls at 0;
//   per-element chunk: F0_i = 2^(Ls + c_i), F1 = 1, lam = 2^(Ls + c_last),
//     then Ls = 0;
//   F2_j = c_j, F3_j = s_j; meta = {mode, resc, lam, Ls after the chunk}.
// ---------------------------------------------------------------------------
template <int NH> struct WalkLds {
    static constexpr int SO = 4;                         // operand slots (chunks k .. k + 3)
    static constexpr int SX = 6;                         // x + record slots (k - 1 .. k + 4)
    static constexpr int SF = 4;                         // factor slots (k - 1 .. k + 2)
    static constexpr int kXHead = 5120;                  // per head: x tile (4 KiB) + record copy (1 KiB)
    static constexpr int kFHead = 528;                   // per head: F0..F3 (32 floats each) + meta
    static constexpr int kOps = 0;
    static constexpr int kX = kOps + SO * kOpsBytes;
    static constexpr int kF = kX + SX * NH * kXHead;
    static constexpr int kBytes = kF + SF * NH * kFHead;
    static_assert(kBytes <= 160 * 1024, "LDS");
};
constexpr int kModeFast = 0, kModeRescale = 1, kModeElem = 2;

template <int NH, bool OPTS, bool HAS_D>
__global__ __launch_bounds__(64 * (2 * NH + 1)) void k_ssd_walk(
    const bf16 *__restrict__ x, const unsigned char *__restrict__ ops, const float *__restrict__ rec,
    const float *__restrict__ D, const float *init, bf16 *__restrict__ y, float *fin, int L, int H, int G,
    int nblk) {
    using Lay = WalkLds<NH>;
    constexpr int NW = 2 * NH;                            // compute waves
    constexpr int RF = Rec<OPTS>::kFloats, RP = Rec<OPTS>::kPieces;
    constexpr int NI = kInsOps + NH * (kInsX + 1);        // copies per chunk
    static_assert(2 * NI < 64, "vmcnt is 6 bits");
    __shared__ __attribute__((aligned(16))) unsigned char smem[Lay::kBytes];

    const int nunits = H / NH;
    const int item = (int)xcd_remap(blockIdx.x, gridDim.x);
    const int b = item / nunits, h0 = (item - b * nunits) * NH;
    const int grp = h0 / (H / G);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const uint32_t smem_lds = lds_addr(smem);
    auto x_slot = [&](int m) { return Lay::kX + (m % Lay::SX) * NH * Lay::kXHead; };
    auto f_slot = [&](int m) { return Lay::kF + (m & (Lay::SF - 1)) * NH * Lay::kFHead; };
    auto o_slot = [&](int m) { return Lay::kOps + (m & (Lay::SO - 1)) * kOpsBytes; };

    if (wave == NW) {
        // ---------------- copy wave ----------------
        const unsigned char *ops_b = ops + ((int64_t)b * nblk * G + grp) * kOpsBytes;
        const int64_t ops_step = (int64_t)G * kOpsBytes, x_step = (int64_t)kBlk * H * 128,
                      rec_step = (int64_t)H * RF * 4;
        const unsigned char *x_b = (const unsigned char *)(x + ((int64_t)b * L * H + h0) * 64);
        const unsigned char *rec_b = (const unsigned char *)(rec + ((int64_t)b * nblk * H + h0) * RF);
        const XOffsets xo_full = x_offsets(lane, kBlk - 1, H);
        const XOffsets xo_tail = x_offsets(lane, L - (nblk - 1) * kBlk - 1, H);
        const uint32_t lane16 = 16u * (uint32_t)lane, recoff = 16u * (uint32_t)min(lane, RP - 1);
        // chunk m's copies; past the last chunk the sources repeat it (into
        // slots nobody reads) so every chunk issues exactly NI copies
        auto issue_ops = [&](int m) {
            const unsigned char *src = ops_b + (int64_t)min(m, nblk - 1) * ops_step;
            const uint32_t dst = smem_lds + (uint32_t)o_slot(m);
            dma16<4>(lane16, src, dst);
            dma16<4>(lane16, src + 4096, dst + 4096);
            dma16<4>(lane16, src + 8192, dst + 8192);
            dma16<4>(lane16, src + 12288, dst + 12288);
            dma16<2>(lane16, src + 16384, dst + 16384);
            static_assert(kInsOps == 18, "operand copies");
        };
        auto issue_x = [&](int m) {
            const int mc = min(m, nblk - 1);
            const XOffsets &xo = mc == nblk - 1 ? xo_tail : xo_full;
            const uint32_t dst = smem_lds + (uint32_t)x_slot(m);
#pragma unroll
            for (int hh = 0; hh < NH; ++hh)
                dma16_4v(xo.v[0], xo.v[1], xo.v[2], xo.v[3], x_b + hh * 128 + mc * x_step - kXBias,
                         dst + hh * Lay::kXHead);
#pragma unroll
            for (int hh = 0; hh < NH; ++hh)  // last: the waits below count from these
                dma16<1>(recoff, rec_b + hh * RF * 4 + mc * rec_step, dst + hh * Lay::kXHead + 4096);
        };
        // lanes 32 hh + j: step j of head hh (NH = 1: lanes 32..63 repeat 0..31)
        const int hh = NH == 2 ? lane >> 5 : 0, j = lane & 31;
        const bool writer = NH == 2 || lane < 32;
        float Ls = 0.f;
        auto factors = [&](int m) {
            const float *rc = (const float *)(smem + x_slot(m) + hh * Lay::kXHead + 4096);
            const float c = rc[j];
            const f32x4 meta = *(const f32x4 *)(rc + 32);
            const float s = OPTS ? rc[36 + j] : 1.f;
            const float cl = meta[0], cmin = meta[1], cmax = meta[2];
            const bool inr = Ls + cmin >= -kRange && Ls + cmax <= kRange;
            const bool alone = cmin >= -kRange && cmax <= kRange;
            const bool fast = inr || alone;
            const float Lb = fast && !inr ? 0.f : Ls;
            const float e_dn = exp2_raw(-(Lb + c)), e_up = exp2_raw(Lb + c);
            float *fd = (float *)(smem + f_slot(m) + hh * Lay::kFHead);
            if (writer) {
                fd[j] = fast ? e_dn * s : e_up;
                fd[32 + j] = fast ? e_up : 1.f;
                fd[64 + j] = c;
                fd[96 + j] = s;
                if (j == 0)
                    *(f32x4 *)(fd + 128) = f32x4{(float)(fast ? (inr ? kModeFast : kModeRescale) : kModeElem),
                                                 fast && !inr ? exp2_raw(Ls) : 1.f, exp2_raw(Ls + cl),
                                                 fast ? Lb + cl : 0.f};
            }
            Ls = fast ? Lb + cl : 0.f;
        };
        // before the first barrier: operands of chunks 0 .. 2, x and records
        // of 0 .. 3 (issued as the iterations -4 .. -1 of the loop below
        // would), factors of chunks 0 and 1
        issue_x(0);
        issue_ops(0);
        issue_x(1);
        issue_ops(1);
        issue_x(2);
        issue_ops(2);
        issue_x(3);
        wait_vm<2 * NI>();  // the record of chunk 1 and everything before it
        factors(0);
        factors(1);
        lds_barrier();
        for (int k = 0; k < nblk; ++k) {
            // slots of chunk k - 1 (operands) and k - 2 (x) are free now
            issue_ops(k + 3);
            issue_x(k + 4);
            // the record of chunk k + 2 (and with it the operands of k + 1
            // and the x tiles of k + 2) was issued two chunks ago
            wait_vm<2 * NI>();
            if (k + 2 < nblk) factors(k + 2);
            if (k + 1 < nblk) lds_barrier();
        }
        wait_vm<0>();  // no copy may land after the workgroup ends
        return;
    }

    // ---------------- compute waves ----------------
    const int hh = wave >> 1, h = h0 + hh;
    const int r = lane & 15, gq = lane >> 4;
    const int ct0 = (wave & 1) * 2;  // first column tile of this wave
    const int xh = hh * Lay::kXHead, fh = hh * Lay::kFHead;

    // g[n][p] with lane (r, gq) of acc_h[nt][ct] holding n = 16 nt + 4 gq + e,
    // p = 16 (ct0 + ct) + r
    f32x4 acc_h[8][2];
    if (init) {
        const float *ib = init + ((int64_t)(b * H + h) * 64) * 128;
#pragma unroll
        for (int nt = 0; nt < 8; ++nt)
#pragma unroll
            for (int ct = 0; ct < 2; ++ct)
                acc_h[nt][ct] = *(const f32x4 *)(ib + (16 * (ct0 + ct) + r) * 128 + 16 * nt + 4 * gq);
    } else {
#pragma unroll
        for (int nt = 0; nt < 8; ++nt)
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) acc_h[nt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const float Dh = HAS_D ? D[h] : 0.f;
    const auto rsY = buf_rsrc(y + ((int64_t)b * L * H + h) * 64, (uint32_t)(((int64_t)(L - 1) * H + 1) * 64 * 2));

    // the state as the bf16 operand of the output product:
    // hB[s][ct] = g[n in 32 s + kset(gq)][p = 16 (ct0 + ct) + r]
    auto state_operand = [&](bf16x8 (&hB)[4][2]) {
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int ct = 0; ct < 2; ++ct)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    hB[s][ct][e] = (bf16)acc_h[2 * s][ct][e];
                    hB[s][ct][e + 4] = (bf16)acc_h[2 * s + 1][ct][e];
                }
    };
    // acc_y[ct][rt] = C_rt g: lane (r, gq) holds y[i = 16 rt + r][p = 16 (ct0 + ct) + 4 gq + e]
    auto state_output = [&](const unsigned char *os, const bf16x8 (&hB)[4][2], f32x4 (&acc_y)[2][2]) {
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) acc_y[ct][0] = acc_y[ct][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const bf16x8 cf = *(const bf16x8 *)(os + (rt * 4 + s) * 1024 + 16 * lane);
#pragma unroll
                for (int ct = 0; ct < 2; ++ct) acc_y[ct][rt] = mfma_bf16(hB[s][ct], cf, acc_y[ct][rt]);
            }
    };
    // E = F0 x of chunk m (the fast path's scaled input), as the B operand
    auto scaled_x = [&](int m, bf16x8 (&V)[2]) {
        const float *F0 = (const float *)(smem + f_slot(m) + fh);
        const f32x4 ea = *(const f32x4 *)(F0 + 4 * gq), eb = *(const f32x4 *)(F0 + 16 + 4 * gq);
        const unsigned char *xt = smem + x_slot(m) + xh;
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
            const bf16x8 X = x_frag(xt, 16 * (ct0 + ct), lane);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                V[ct][e] = (bf16)((float)X[e] * ea[e]);
                V[ct][e + 4] = (bf16)((float)X[e + 4] * eb[e]);
            }
        }
    };
    // fast chunk: acc_y = C g + (C B^T) E, g += B^T E
    auto chunk_fast = [&](int m, const bf16x8 (&V)[2], f32x4 (&acc_y)[2][2]) {
        const unsigned char *os = smem + o_slot(m);
        bf16x8 hB[4][2];
        state_operand(hB);
        state_output(os, hB, acc_y);
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            const bf16x8 gf = *(const bf16x8 *)(os + kOffG + rt * 1024 + 16 * lane);
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) acc_y[ct][rt] = mfma_bf16(V[ct], gf, acc_y[ct][rt]);
        }
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) {
            const bf16x8 bt = *(const bf16x8 *)(os + kOffBt + nt * 1024 + 16 * lane);
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) acc_h[nt][ct] = mfma_bf16(bt, V[ct], acc_h[nt][ct]);
        }
    };
    // per-element chunk (every exponent <= 0 for a non-increasing prefix):
    //   y = 2^(Ls + c_i) C_i g + (mask . C B^T) x,  mask_ij = 2^(c_i - c_j) s_j [j <= i],
    //   g' = 2^(Ls + c_last) g + B^T U,  U_j = 2^(c_last - c_j) s_j x_j
    auto chunk_elem = [&](int m, f32x4 (&acc_y)[2][2]) {
        const unsigned char *os = smem + o_slot(m);
        const float *fb = (const float *)(smem + f_slot(m) + fh);
        const float *cc = fb + 64;
        const f32x4 ca = *(const f32x4 *)(cc + 4 * gq), cb = *(const f32x4 *)(cc + 16 + 4 * gq);
        const float ci[2] = {cc[r], cc[16 + r]};
        const float pre[2] = {fb[r], fb[16 + r]};
        const float c_last = cc[31];
        const float lam = rfl(fb[130]);
        f32x4 sa = {1.f, 1.f, 1.f, 1.f}, sb = {1.f, 1.f, 1.f, 1.f};
        if constexpr (OPTS) {
            sa = *(const f32x4 *)(fb + 96 + 4 * gq);
            sb = *(const f32x4 *)(fb + 112 + 4 * gq);
        }
        const unsigned char *xt = smem + x_slot(m) + xh;
        bf16x8 hB[4][2];
        state_operand(hB);
        bf16x8 X[2];
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) X[ct] = x_frag(xt, 16 * (ct0 + ct), lane);
        state_output(os, hB, acc_y);
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) acc_y[ct][rt] *= pre[rt];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            const int i = 16 * rt + r;
            bf16x8 gm = *(const bf16x8 *)(os + kOffG + rt * 1024 + 16 * lane);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                // above the diagonal the tile is zero; its exponent is replaced so
                // that no factor overflows (a select, not a branch)
                const int ja = 4 * gq + e, jb = 16 + 4 * gq + e;
                const float fa = exp2_raw(ja <= i ? ci[rt] - ca[e] : -256.f) * sa[e];
                const float fb2 = exp2_raw(jb <= i ? ci[rt] - cb[e] : -256.f) * sb[e];
                gm[e] = (bf16)((float)gm[e] * fa);
                gm[e + 4] = (bf16)((float)gm[e + 4] * fb2);
            }
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) acc_y[ct][rt] = mfma_bf16(X[ct], gm, acc_y[ct][rt]);
        }
        bf16x8 U[2];
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                U[ct][e] = (bf16)((float)X[ct][e] * exp2_raw(c_last - ca[e]) * sa[e]);
                U[ct][e + 4] = (bf16)((float)X[ct][e + 4] * exp2_raw(c_last - cb[e]) * sb[e]);
            }
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) {
            const bf16x8 bt = *(const bf16x8 *)(os + kOffBt + nt * 1024 + 16 * lane);
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) acc_h[nt][ct] = mfma_bf16(bt, U[ct], acc_h[nt][ct] * lam);
        }
    };
    // y of chunk m = F1_i acc_y + D x, to bf16; lane groups gq, gq ^ 1 swap one
    // 8-byte piece (one permlane16 swap per dword) so each holds 8 consecutive
    // columns of its row: one 16-byte store per row tile
    auto store_y = [&](int m, const f32x4 (&acc_y)[2][2]) {
        const float *F1 = (const float *)(smem + f_slot(m) + fh) + 32;
        const float rs[2] = {F1[r], F1[16 + r]};
        const unsigned char *xt = smem + x_slot(m) + xh;
        const int t0 = m * kBlk;
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            const int i = 16 * rt + r;
            uint32_t pk[2][2];
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
                f32x4 v = acc_y[ct][rt] * rs[rt];
                if constexpr (HAS_D) {
                    const u32x2 xr = x_row4(xt, i, 16 * (ct0 + ct) + 4 * gq);
                    v[0] += Dh * bf16_lo(xr[0]);
                    v[1] += Dh * bf16_hi(xr[0]);
                    v[2] += Dh * bf16_lo(xr[1]);
                    v[3] += Dh * bf16_hi(xr[1]);
                }
                pk[ct][0] = pack_bf16x2(v[0], v[1]);
                pk[ct][1] = pack_bf16x2(v[2], v[3]);
            }
            const bool odd = gq & 1;
            const uint32_t off_row = (t0 + i < L) ? (uint32_t)(t0 + i) * (uint32_t)H * 128u : kBufOff;
            // lane group gq even ends with columns 16 ct0 + 8 (gq / 2) .. + 7,
            // odd with 16 (ct0 + 1) + 8 (gq / 2) .. + 7
            const auto s0 = __builtin_amdgcn_permlane16_swap(pk[0][0], pk[1][0], false, false);
            const auto s1 = __builtin_amdgcn_permlane16_swap(pk[0][1], pk[1][1], false, false);
            const u32x4 out = {s0[0], s1[0], s0[1], s1[1]};
            const int col = 16 * (ct0 + (odd ? 1 : 0)) + 8 * (gq >> 1);
            buf_st16(out, rsY, off_row == kBufOff ? kBufOff : off_row + (uint32_t)col * 2u);
        }
    };

    lds_barrier();  // operands of chunk 0, x and factors of chunks 0 and 1
    bf16x8 Vc[2];
    scaled_x(0, Vc);
    // chunk k: its state products, its output (overlapping the state update)
    // and the scaled x of chunk k + 1, which does not depend on them
    for (int k = 0; k < nblk; ++k) {
        const f32x4 meta = *(const f32x4 *)(smem + f_slot(k) + fh + 512);
        const int mode = (int)rfl(meta[0]);
        f32x4 acc_y[2][2];
        // each branch is one straight-line block, so the output and the next
        // scaled x (past the last chunk: unused values from a stale slot) can
        // be scheduled between the state products
        if (mode == kModeElem) {
            chunk_elem(k, acc_y);
            store_y(k, acc_y);
            scaled_x(k + 1, Vc);
        } else {
            if (mode == kModeRescale) {
                const float sc = rfl(meta[1]);
#pragma unroll
                for (int nt = 0; nt < 8; ++nt)
#pragma unroll
                    for (int ct = 0; ct < 2; ++ct) acc_h[nt][ct] *= sc;
            }
            chunk_fast(k, Vc, acc_y);
            store_y(k, acc_y);
            scaled_x(k + 1, Vc);
        }
        if (k + 1 < nblk) lds_barrier();
    }

    if (fin) {
        const float sc = exp2_raw(rfl(((const float *)(smem + f_slot(nblk - 1) + fh))[131]));
        float *fb = fin + ((int64_t)(b * H + h) * 64) * 128;
#pragma unroll
        for (int nt = 0; nt < 8; ++nt)
#pragma unroll
            for (int ct = 0; ct < 2; ++ct)
                *(f32x4 *)(fb + (16 * (ct0 + ct) + r) * 128 + 16 * nt + 4 * gq) = acc_h[nt][ct] * sc;
    }
}

bool walk_supported(const Dims &d) {
    if (!(d.dtype == 1 && d.P == 64 && d.N == 128 && d.L >= 1 && d.b >= 1)) return false;
    // y offsets inside one (b, h) walk and the grid are 32-bit
    const int64_t lim = (int64_t)1 << 31;
    return d.L * d.H * d.P * 2 < lim && d.b * d.H < lim && d.b * d.L * d.H < lim;
}

WalkBytes walk_bytes(const Dims &d) {
    const int64_t nblk = (d.L + kBlk - 1) / kBlk;
    WalkBytes w;
    w.ops = d.b * nblk * d.G * kOpsBytes;
    w.rec = d.b * nblk * d.H * Rec<true>::kFloats * 4;  // sized for either record form
    return w;
}

hipError_t launch_walk_prep(const Dims &d, const void *dt, const float *A, const void *B, const void *C,
                            void *ops, float *rec, hipStream_t st, const DtOpts *o) {
    const int nblk = (int)((d.L + kBlk - 1) / kBlk);
    dim3 grid((unsigned)(d.b * nblk), (unsigned)(d.G + 1));
    if (o)
        k_walk_prep<true><<<grid, 256, 0, st>>>((const bf16 *)B, (const bf16 *)C, (const bf16 *)dt, A,
                                                (unsigned char *)ops, rec, (int)d.L, (int)d.H, (int)d.G, nblk, *o);
    else
        k_walk_prep<false><<<grid, 256, 0, st>>>((const bf16 *)B, (const bf16 *)C, (const bf16 *)dt, A,
                                                 (unsigned char *)ops, rec, (int)d.L, (int)d.H, (int)d.G, nblk,
                                                 DtOpts{nullptr, 0.f, 0.f, 0, 0});
    return hipGetLastError();
}

namespace {
template <int NH, bool OPTS, bool HAS_D>
void launch_walk_t(const Dims &d, const void *x, const void *ops, const float *rec, const float *D,
                   const float *init, void *y, float *fin, hipStream_t st) {
    const int nblk = (int)((d.L + kBlk - 1) / kBlk);
    k_ssd_walk<NH, OPTS, HAS_D><<<(unsigned)(d.b * (d.H / NH)), 64 * (2 * NH + 1), 0, st>>>(
        (const bf16 *)x, (const unsigned char *)ops, rec, D, init, (bf16 *)y, fin, (int)d.L, (int)d.H, (int)d.G,
        nblk);
}
template <int NH>
void launch_walk_nh(const Dims &d, const void *x, const void *ops, const float *rec, const float *D,
                    const float *init, void *y, float *fin, hipStream_t st, bool opts) {
    if (opts) {
        if (D) launch_walk_t<NH, true, true>(d, x, ops, rec, D, init, y, fin, st);
        else launch_walk_t<NH, true, false>(d, x, ops, rec, D, init, y, fin, st);
    } else {
        if (D) launch_walk_t<NH, false, true>(d, x, ops, rec, D, init, y, fin, st);
        else launch_walk_t<NH, false, false>(d, x, ops, rec, D, init, y, fin, st);
    }
}
}  // namespace

hipError_t launch_walk_main(const Dims &d, const void *x, const void *ops, const float *rec, const float *D,
                            const float *init, void *y, float *fin, hipStream_t st, bool opts) {
    // One head per workgroup while every (b, h) gets a CU of its own (256 on
    // gfx950); beyond that, two heads per workgroup share each chunk's operand
    // copies when both belong to one group.  Measured on MI355X: batch 8 x 32
    // heads (256 walks) 78 us with one head per workgroup against 84 us with
    // two; batch 4 x 80 heads 162 us with two against 265 us with one.
    constexpr int64_t kCUs = 256;
    if ((d.H / d.G) % 2 == 0 && d.b * d.H > kCUs) launch_walk_nh<2>(d, x, ops, rec, D, init, y, fin, st, opts);
    else launch_walk_nh<1>(d, x, ops, rec, D, init, y, fin, st, opts);
    return hipGetLastError();
}

}  // namespace ssd
