// Device-side helpers shared by the SSD kernels (gfx950 / CDNA4 only).
//
// MFMA conventions used throughout (16 x 16 output tiles, wave64):
//   lane l, r = l % 16, g = l / 16 (0..3)
//   A operand: lane holds A[m = r][k in kset(g)]
//   B operand: lane holds B[k in kset(g)][n = r]
//   D (4 x f32 per lane): D[m = 4 g + e][n = r], e = 0..3
// v_mfma_f32_16x16x32_bf16 takes 8 k-values per lane and v_mfma_f32_16x16x4_f32
// one.  The order of k inside a lane group never matters for a contraction as
// long as A and B use the same kset(g); the kernels pick contiguous sets
// (bf16: k = 8 g .. 8 g + 7) so fragments load as one 16-byte vector.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 v) { return (float)v; }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) { return (bf16)v; }

__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ u32x4 as_u32x4(bf16x8 v) { return __builtin_bit_cast(u32x4, v); }

// 16-byte fragments for either element type.  A lane holds KPL consecutive
// values of the contraction index (bf16: 8, one 16x16x32 MFMA; f32: 4, four
// 16x16x4 MFMAs, the e-th taking element e), so a fragment step covers KSTEP
// = 4 KPL values of k across the four lane groups.
template <typename T> struct Frag {
    static constexpr int KPL = 16 / (int)sizeof(T);
    static constexpr int KSTEP = 4 * KPL;
};

template <typename T>
__device__ __forceinline__ f32x4 mma16(u32x4 a, u32x4 b, f32x4 c) {
    if constexpr (sizeof(T) == 2) {
        return mfma_bf16(as_bf16x8(a), as_bf16x8(b), c);
    } else {
        // Each element goes through a scalar first: clang's __builtin_bit_cast of an
        // ext-vector element expression reads element 0 whatever the index.
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t ua = a[e], ub = b[e];
            c = mfma_f32(__builtin_bit_cast(float, ua), __builtin_bit_cast(float, ub), c);
        }
        return c;
    }
}

// Every element of a fragment times s (bf16: rounded back to bf16).
template <typename T>
__device__ __forceinline__ u32x4 frag_scale(u32x4 v, float s) {
    if constexpr (sizeof(T) == 2) {
        bf16x8 t = as_bf16x8(v);
#pragma unroll
        for (int e = 0; e < 8; ++e) t[e] = (bf16)((float)t[e] * s);
        return as_u32x4(t);
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t u = v[e];
            v[e] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(float, u) * s);
        }
        return v;
    }
}

// A fragment from KPL float32 values base[0], base[ld], base[2 ld], ...
// (a column of a row-major float32 matrix), converted to T.
template <typename T>
__device__ __forceinline__ u32x4 frag_from_f32_col(const float *base, int64_t ld) {
    if constexpr (sizeof(T) == 2) {
        bf16x8 t;
#pragma unroll
        for (int e = 0; e < 8; ++e) t[e] = (bf16)base[e * ld];
        return as_u32x4(t);
    } else {
        u32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float f = base[e * ld];
            v[e] = __builtin_bit_cast(uint32_t, f);
        }
        return v;
    }
}

// Step-size preprocessing and input scaling (Mamba review, section 3.1: the
// step size is a softplus of a linear map of the input, whose bias is
// dt_bias; section 2.2 and guide equation (2): the zero-order-hold input
// factor is the integral of exp(u A) over the step; section 3.3: the Euler
// factor is the step itself).
struct DtOpts {
    const float *bias;  // [H] or null
    float lo, hi;       // clamp to [lo, hi] when hi > lo, after softplus
    int softplus;       // nonzero: softplus(dt + bias)
    int scale;          // 0: x as is, 1: dt x (Euler), 2: expm1(dt A) / A x (zero-order hold)
};

__device__ __forceinline__ float dt_effective(float raw, int h, const DtOpts &o) {
    float v = raw + (o.bias ? o.bias[h] : 0.f);
    if (o.softplus) v = v > 20.f ? v : log1pf(expf(v));
    if (o.hi > o.lo) v = fminf(fmaxf(v, o.lo), o.hi);
    return v;
}

__device__ __forceinline__ float input_scale(float d, float Ah, int scale) {
    if (scale == 1) return d;
    if (scale == 2) return Ah != 0.f ? expm1f(d * Ah) / Ah : d;
    return 1.f;
}

// Blocks are dealt to the 8 XCDs round-robin (block k runs on XCD k % 8), and
// each XCD has its own L2.  Work items that share operands (all heads of one
// chunk share C, B and C B^T) should land on the same XCD, so map block k to
// a contiguous slice of work items per XCD.  Identity when the count is not a
// multiple of 8.
__device__ __forceinline__ int64_t xcd_remap(int64_t bid, int64_t total) {
    if (total % 8 != 0) return bid;
    const int64_t per = total / 8;
    return (bid % 8) * per + bid / 8;
}

// s_waitcnt immediate that waits for lgkmcnt 0 (LDS and scalar memory) and
// leaves the vector-memory and export counters at their maxima.
constexpr int kWaitScalar = 0xC07F;

// Workgroup barrier for LDS hand-offs only: waits for this wave's LDS
// operations (and scalar loads) and meets the other waves, without the
// release fence of __syncthreads, which would also wait for every global
// load in flight and defeat a prefetch of later operands.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(kWaitScalar);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);  // compiler-only: memory accesses stay on their side
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Direct global-to-LDS copy of 16 bytes per lane (global_load_lds_dwordx4):
// lane l's bytes land at dst_wave_base + 16 l (dst_wave_base is uniform).
// The copy counts in vmcnt like a load and bypasses the registers.
__device__ __forceinline__ void copy16_to_lds(const void *src, void *dst_wave_base) {
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)src,
                                     (__attribute__((address_space(3))) void *)dst_wave_base, 16, 0, 0);
}


// Row-major bf16 tiles filled by direct copies and read with transposing
// reads use a pair swizzle: the 32-byte pair p of row r (16-byte chunks 2 p,
// 2 p + 1) is stored at pair p ^ (tr_swz(r) & (pairs per row - 1)).  A
// transposing read touches rows r0 + 8 grp + m (m < 4, grp < 4) at one pair;
// tr_swz mixes the row bits that vary there (0, 1, 3, 4) so those 16 rows
// fall on every 32-byte bank slot of a 256-byte window at most twice.
__device__ __forceinline__ int tr_swz(int row) {
    return (((row >> 3) & 3) ^ (((row >> 1) & 1) << 1)) | ((row & 1) << 2);
}

template <int ROWB>
__device__ __forceinline__ int tr_chunk_slot(int row, int chunk) {
    constexpr int NP = ROWB / 32;  // 32-byte pairs per row
    if constexpr (NP <= 1) return chunk;
    else return (((chunk >> 1) ^ (tr_swz(row) & (NP - 1))) << 1) | (chunk & 1);
}

typedef short i16x4 __attribute__((ext_vector_type(4)));

// ds_read_b64_tr_b16: in each 16-lane group, lane j points at the 4-element
// piece (row r0 + j / 4, columns c0 + 4 (j % 4) ..) and receives column
// c0 + j of rows r0 .. r0 + 3.
template <int ROWB>
__device__ __forceinline__ i16x4 read_tr4(const unsigned char *tile, int r0, int c0, int lane) {
    const int j = lane & 15;
    const int row = r0 + (j >> 2);
    const int col = c0 + 4 * (j & 3);                    // first element of this lane's piece
    const int slot = tr_chunk_slot<ROWB>(row, col >> 3);
    const unsigned char *a = tile + row * ROWB + slot * 16 + ((col >> 2) & 1) * 8;
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4 *)a);
}

// MFMA fragment (8 steps k0 + 8 grp .. + 7 of column c0 + r) from a row-major tile
template <int ROWB>
__device__ __forceinline__ bf16x8 frag_tr(const unsigned char *tile, int k0, int c0, int lane) {
    const int grp = lane >> 4;
    const i16x4 lo = read_tr4<ROWB>(tile, k0 + 8 * grp, c0, lane);
    const i16x4 hi = read_tr4<ROWB>(tile, k0 + 8 * grp + 4, c0, lane);
    bf16x8 f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const short a = lo[e], b = hi[e];
        f[e] = __builtin_bit_cast(bf16, a);
        f[e + 4] = __builtin_bit_cast(bf16, b);
    }
    return f;
}

// The same fragment through a per-lane byte offset computed once: for k0 a
// multiple of 32 the lane's rows k0 + 8 grp + 4 h + j / 4 have the same
// swizzle for every k0 and h, so only (k0 + 4 h) * ROWB changes (an
// immediate offset of the LDS read).  c0 is a multiple of 16.
template <int ROWB>
__device__ __forceinline__ int tr_lane_offset(int c0, int lane) {
    const int j = lane & 15, grp = lane >> 4;
    const int row = 8 * grp + (j >> 2);
    const int col = c0 + 4 * (j & 3);
    return row * ROWB + tr_chunk_slot<ROWB>(row, col >> 3) * 16 + ((col >> 2) & 1) * 8;
}

template <int ROWB>
__device__ __forceinline__ bf16x8 frag_tr_off(const unsigned char *tile, int k0, int off) {
    const unsigned char *a = tile + off + k0 * ROWB;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4 *)a);
    const i16x4 hi =
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4 *)(a + 4 * ROWB));
    bf16x8 f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const short a0 = lo[e], b0 = hi[e];
        f[e] = __builtin_bit_cast(bf16, a0);
        f[e + 4] = __builtin_bit_cast(bf16, b0);
    }
    return f;
}

// Four consecutive elements (col % 4 == 0) of row `row` of such a tile.
template <int ROWB>
__device__ __forceinline__ u32x2 lds_row4(const unsigned char *tile, int row, int col) {
    const int slot = tr_chunk_slot<ROWB>(row, col >> 3);
    return *(const u32x2 *)(tile + row * ROWB + slot * 16 + ((col >> 2) & 1) * 8);
}

// Copy rows 0 .. nrows - 1 (row index clamped to nvalid - 1) of a bf16 tile with
// rows of ROWB bytes at global row stride ld (elements) into LDS with the pair
// swizzle; copies k = wave, wave + NW, ... of 1 KiB each (NW waves).
template <int ROWB, int NW>
__device__ __forceinline__ void copy_tile_to_lds(const bf16 *__restrict__ src, int64_t ld, int nrows,
                                                 int nvalid, unsigned char *dst, int wave, int lane) {
    constexpr int CPR = ROWB / 16, RPC = 1024 / ROWB;
    const int ncopies = nrows * ROWB / 1024;
    for (int k = wave; k < ncopies; k += NW) {
        const int row = k * RPC + lane / CPR;
        const int chunk = tr_chunk_slot<ROWB>(row, lane % CPR);  // the swizzle is an involution
        const bf16 *g = src + (int64_t)min(row, nvalid - 1) * ld + chunk * 8;
        copy16_to_lds(g, dst + k * 1024);
    }
}

// Buffer resource over [base, base + bytes), bytes < 2^31.  A load at an
// offset at or past `bytes` returns zero and a store there is dropped, so a
// lane is switched off by giving it the offset kBufOff: no branch, and the
// instruction counts in vmcnt like every other, which keeps the compiler's
// counted waits exact across a loop.
constexpr uint32_t kBufOff = 0x80000000u;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             0x00020000);
}
__device__ __forceinline__ u32x4 buf_ld16(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(rs, (int)off, 0, 0);
}
// The same with a wave-uniform part of the offset in soff (a scalar register):
// a lane switched off by voff = kBufOff stays past the end whether or not the
// hardware counts soff in its range check (soff stays below 2^31).
__device__ __forceinline__ u32x4 buf_ld16s(__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b128(rs, (int)voff, (int)soff, 0);
}
__device__ __forceinline__ u32x2 buf_ld8(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b64(rs, (int)off, 0, 0);
}
__device__ __forceinline__ float buf_ldf(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, (int)off, 0, 0));
}
__device__ __forceinline__ uint16_t buf_ld2(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b16(rs, (int)off, 0, 0);
}
__device__ __forceinline__ void buf_st2(uint16_t v, __amdgpu_buffer_rsrc_t rs, uint32_t off) {
    __builtin_amdgcn_raw_buffer_store_b16(v, rs, (int)off, 0, 0);
}
__device__ __forceinline__ void buf_st8(u32x2 v, __amdgpu_buffer_rsrc_t rs, uint32_t off) {
    __builtin_amdgcn_raw_buffer_store_b64(v, rs, (int)off, 0, 0);
}
__device__ __forceinline__ void buf_st16(u32x4 v, __amdgpu_buffer_rsrc_t rs, uint32_t off) {
    __builtin_amdgcn_raw_buffer_store_b128(v, rs, (int)off, 0, 0);
}

// Four rows r0..r0+3 of 8 bf16 columns c0..c0+7 (v[k] = row r0 + k) stored
// transposed, dst[c * dstride + r]: a register transpose with byte permutes
// and eight 8-byte LDS stores.
// Column c goes to LDS row rowof(c) (the identity unless a caller permutes).
struct RowIdentity {
    __device__ int operator()(int c) const { return c; }
};
template <typename RowOf = RowIdentity>
__device__ __forceinline__ void write_transposed_4x8(const u32x4 (&v)[4], bf16 *dst, int dstride,
                                                     int r0, int c0, RowOf rowof = RowOf{}) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        // dword m of each row holds columns c0 + 2m (low half) and c0 + 2m + 1 (high half)
        const uint32_t lo01 = __builtin_amdgcn_perm(v[1][m], v[0][m], 0x05040100u);
        const uint32_t lo23 = __builtin_amdgcn_perm(v[3][m], v[2][m], 0x05040100u);
        const uint32_t hi01 = __builtin_amdgcn_perm(v[1][m], v[0][m], 0x07060302u);
        const uint32_t hi23 = __builtin_amdgcn_perm(v[3][m], v[2][m], 0x07060302u);
        *(u32x2 *)(dst + rowof(c0 + 2 * m) * dstride + r0) = u32x2{lo01, lo23};
        *(u32x2 *)(dst + rowof(c0 + 2 * m + 1) * dstride + r0) = u32x2{hi01, hi23};
    }
}

// Copy a [rows x cols] bf16 tile from global memory (row stride `ld`
// elements) into LDS transposed: dst[c * dstride + r] = src[r * ld + c],
// optionally times scale[r] (rounded back to bf16).  Rows >= nvalid read as
// zero.  rows % 4 == 0, cols % 8 == 0, dstride % 4 == 0.  Each thread moves
// 4 x 8 blocks: four 16-byte loads, a register transpose with byte
// permutes, eight 8-byte LDS stores.
template <bool SCALE>
__device__ __forceinline__ void stage_transposed_bf16(const bf16 *__restrict__ src, int64_t ld,
                                                      int rows, int cols, int nvalid,
                                                      bf16 *dst, int dstride,
                                                      const float *scale) {
    const int nbc = cols / 8, nbr = rows / 4;
    for (int blk = threadIdx.x; blk < nbr * nbc; blk += blockDim.x) {
        const int br = blk / nbc, bc = blk - br * nbc;
        const int r0 = br * 4, c0 = bc * 8;
        u32x4 v[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int r = r0 + k;
            if (r < nvalid) {
                v[k] = *(const u32x4 *)(src + (int64_t)r * ld + c0);
                if constexpr (SCALE) {
                    bf16x8 t = as_bf16x8(v[k]);
                    const float w = scale[r];
#pragma unroll
                    for (int e = 0; e < 8; ++e) t[e] = (bf16)((float)t[e] * w);
                    v[k] = as_u32x4(t);
                }
            } else {
                v[k] = u32x4{0u, 0u, 0u, 0u};
            }
        }
        write_transposed_4x8(v, dst, dstride, r0, c0);
    }
}

// The same transposed copy for NROWS rows and COLS columns known at compile
// time, by NT threads, reading through a buffer resource: row r starts at
// byte r * ldb from the resource base, and rows at or past nvalid read as
// zero.  In two steps, so that a caller can issue other loads between them:
// load() issues every load (none behind a branch), write() stores to LDS
// once they have landed.
template <int NROWS, int COLS, int NT>
struct TrStage {
    static constexpr int NBC = COLS / 8, NB = (NROWS / 4) * NBC, IT = (NB + NT - 1) / NT;
    u32x4 v[IT][4];
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, uint32_t ldb, int nvalid) {
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int blk = (int)threadIdx.x + it * NT;
            const int br = blk / NBC, bc = blk - br * NBC;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int r = 4 * br + k;
                v[it][k] = buf_ld16(rs, (blk < NB && r < nvalid) ? (uint32_t)r * ldb + 16u * bc : kBufOff);
            }
        }
    }
    template <typename RowOf = RowIdentity>
    __device__ __forceinline__ void write(bf16 *dst, int dstride, RowOf rowof = RowOf{}) const {
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int blk = (int)threadIdx.x + it * NT;
            const int br = blk / NBC, bc = blk - br * NBC;
            if (NB % NT == 0 || blk < NB) write_transposed_4x8(v[it], dst, dstride, 4 * br, 8 * bc, rowof);
        }
    }
};

}  // namespace ssd
