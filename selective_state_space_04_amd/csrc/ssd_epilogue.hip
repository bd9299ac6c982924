// Normalisation after the gate (review page, section "Mamba-2 ブロック": one
// normalisation layer after the SSM output is multiplied by the gate and
// before the output projection; Mamba review, section 3.4: the gate is SiLU of
// a second projection z).  Per token, g = y * silu(z) over its H * P channels,
// split into ngroups equal contiguous groups, each scaled to unit root mean
// square and multiplied by a per-channel weight:
//   out = g / sqrt(mean_group(g^2) + eps) * weight
#include "ssd_device.h"
#include "ssd_launch.h"

namespace ssd {

template <typename T> struct Vec8;
template <> struct Vec8<bf16> {
    static __device__ __forceinline__ void unpack(const u32x4 (&w)[1], float *v) {
        const bf16x8 t = as_bf16x8(w[0]);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (float)t[e];
    }
    static __device__ __forceinline__ void pack(const float *v, u32x4 (&w)[1]) {
        bf16x8 t;
#pragma unroll
        for (int e = 0; e < 8; ++e) t[e] = (bf16)v[e];
        w[0] = as_u32x4(t);
    }
    static __device__ __forceinline__ void load(const bf16 *p, float *v) {
        const bf16x8 t = *(const bf16x8 *)p;
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (float)t[e];
    }
    static __device__ __forceinline__ void store(bf16 *p, const float *v) {
        bf16x8 t;
#pragma unroll
        for (int e = 0; e < 8; ++e) t[e] = (bf16)v[e];
        *(bf16x8 *)p = t;
    }
};
template <> struct Vec8<float> {
    static __device__ __forceinline__ void unpack(const u32x4 (&w)[2], float *v) {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = __uint_as_float(w[e >> 2][e & 3]);
    }
    static __device__ __forceinline__ void pack(const float *v, u32x4 (&w)[2]) {
#pragma unroll
        for (int e = 0; e < 8; ++e) w[e >> 2][e & 3] = __float_as_uint(v[e]);
    }
    static __device__ __forceinline__ void load(const float *p, float *v) {
        const f32x4 a = *(const f32x4 *)p, b = *(const f32x4 *)(p + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            v[e] = a[e];
            v[e + 4] = b[e];
        }
    }
    static __device__ __forceinline__ void store(float *p, const float *v) {
        *(f32x4 *)p = f32x4{v[0], v[1], v[2], v[3]};
        *(f32x4 *)(p + 4) = f32x4{v[4], v[5], v[6], v[7]};
    }
};

__device__ __forceinline__ float silu(float z) { return z / (1.f + __expf(-z)); }

// Wider rows or more groups: one workgroup per token row of D = H * P
// channels.  Per group: pass 1 sums
// g^2 over 8-channel pieces (16-byte loads) and reduces across the
// workgroup in a fixed order; pass 2 recomputes g from the same (now cached)
// y and z and writes out.  Each thread rewrites only the pieces it read, so
// out may be y itself.
template <typename T>
__global__ __launch_bounds__(256) void k_gated_rmsnorm(const T *y, const T *__restrict__ z,
                                                       const float *__restrict__ w, T *out,
                                                       int64_t D, int64_t Dg, int ngroups,
                                                       float eps) {
    const int64_t row = blockIdx.x;
    const T *yr = y + row * D;
    const T *zr = z + row * D;
    T *orow = out + row * D;
    __shared__ float red[4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (int gi = 0; gi < ngroups; ++gi) {
        const int64_t base = (int64_t)gi * Dg;
        float ss = 0.f;
        for (int64_t k = base + (int64_t)tid * 8; k < base + Dg; k += 256 * 8) {
            float yv[8], zv[8];
            Vec8<T>::load(yr + k, yv);
            Vec8<T>::load(zr + k, zv);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float g = yv[e] * silu(zv[e]);
                ss += g * g;
            }
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, 64);
        if (lane == 0) red[wave] = ss;
        __syncthreads();
        const float tot = red[0] + red[1] + red[2] + red[3];
        __syncthreads();  // red is reused by the next group
        const float scale = rsqrtf(tot / (float)Dg + eps);
        for (int64_t k = base + (int64_t)tid * 8; k < base + Dg; k += 256 * 8) {
            float yv[8], zv[8], o[8];
            Vec8<T>::load(yr + k, yv);
            Vec8<T>::load(zr + k, zv);
            const f32x4 w0 = *(const f32x4 *)(w + k), w1 = *(const f32x4 *)(w + k + 4);
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] = yv[e] * silu(zv[e]) * scale * (e < 4 ? w0[e] : w1[e - 4]);
            Vec8<T>::store(orow + k, o);
        }
    }
}

// Rows of at most 256 * 8 * MAXP channels and at most 8 groups: one pass.
// One to four waves per row (as few as hold the row at MAXP pieces a
// thread); each thread keeps g for its (up to MAXP) 8-channel pieces in
// registers, accumulates g^2 per group, and after one fixed-order reduction
// per group scales and stores them, so y and z are read once.  Every load
// (y, z and the weight of each piece) is issued before the first is used:
// buffer loads whose pieces past the row get an offset past the resource's
// end (they read zero, give g = 0 and add nothing), so no branch separates
// them and they are all in flight together.  y, z and out stream through
// once (non-temporal); the weight vector is shared by every row and cached.
template <typename T, int MAXP>
__global__ __launch_bounds__(256) void k_gated_rmsnorm_reg(const T *y, const T *__restrict__ z,
                                                           const float *__restrict__ w, T *out,
                                                           int D, int Dg, int ngroups, float eps) {
    constexpr int VW = (int)sizeof(T) / 2;  // 16-byte words per 8-channel piece
    constexpr int kNT = 2;                  // cache-policy operand: non-temporal
    const int64_t row = blockIdx.x;
    const uint32_t rowbytes = (uint32_t)D * (uint32_t)sizeof(T);
    const auto rsY = buf_rsrc(y + row * D, rowbytes);
    const auto rsZ = buf_rsrc(z + row * D, rowbytes);
    const auto rsO = buf_rsrc(out + row * D, rowbytes);
    const auto rsW = buf_rsrc(w, (uint32_t)D * 4u);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nthr = blockDim.x, nwaves = nthr >> 6;
    const int npieces = D / 8;
    u32x4 yw[MAXP][VW], zw[MAXP][VW];
    f32x4 wv[MAXP][2];
#pragma unroll
    for (int u = 0; u < MAXP; ++u) {
        const int pc = tid + nthr * u;
        const bool in = pc < npieces;
#pragma unroll
        for (int v = 0; v < VW; ++v) {
            const uint32_t off = in ? (uint32_t)pc * 8u * (uint32_t)sizeof(T) + 16u * v : kBufOff;
            yw[u][v] = __builtin_amdgcn_raw_buffer_load_b128(rsY, (int)off, 0, kNT);
            zw[u][v] = __builtin_amdgcn_raw_buffer_load_b128(rsZ, (int)off, 0, kNT);
        }
#pragma unroll
        for (int v = 0; v < 2; ++v)
            wv[u][v] = __builtin_bit_cast(f32x4, buf_ld16(rsW, in ? (uint32_t)pc * 32u + 16u * v : kBufOff));
    }
    float g[MAXP][8];
    float ss[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) ss[k] = 0.f;
#pragma unroll
    for (int u = 0; u < MAXP; ++u) {
        float yv[8], zv[8];
        Vec8<T>::unpack(yw[u], yv);
        Vec8<T>::unpack(zw[u], zv);
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            g[u][e] = yv[e] * silu(zv[e]);
            acc += g[u][e] * g[u][e];
        }
        const int gi = (8 * (tid + nthr * u)) / Dg;  // past the row: >= 8, or acc = 0
#pragma unroll
        for (int k = 0; k < 8; ++k) ss[k] += (k == gi) ? acc : 0.f;
    }
    __shared__ float red[4][8];
    float scale[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        if (k < ngroups) {
            float v = ss[k];
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
            if (lane == 0) red[wave][k] = v;
        }
    }
    lds_barrier();
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        float tot = red[0][k];
        for (int wi = 1; wi < nwaves; ++wi) tot += red[wi][k];  // fixed order
        scale[k] = k < ngroups ? rsqrtf(tot / (float)Dg + eps) : 0.f;
    }
#pragma unroll
    for (int u = 0; u < MAXP; ++u) {
        const int pc = tid + nthr * u;
        const int gi = (8 * pc) / Dg;
        float sc = 0.f;
#pragma unroll
        for (int k = 0; k < 8; ++k) sc = (k == gi) ? scale[k] : sc;
        float o[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = g[u][e] * sc * wv[u][e >> 2][e & 3];
        u32x4 ow[VW];
        Vec8<T>::pack(o, ow);
        const uint32_t off = pc < npieces ? (uint32_t)pc * 8u * (uint32_t)sizeof(T) : kBufOff;
#pragma unroll
        for (int v = 0; v < VW; ++v) __builtin_amdgcn_raw_buffer_store_b128(ow[v], rsO, (int)(off + 16u * v), 0, kNT);
    }
}

hipError_t launch_gated_rmsnorm(const Dims &d, int64_t ngroups, float eps, const void *y,
                                const void *z, const float *w, void *out, hipStream_t st) {
    const int64_t rows = d.b * d.L, D = d.H * d.P;
    if (rows == 0 || D == 0) return hipSuccess;
    // 8-channel pieces per thread: 4, 5 or 8, whichever leaves the fewest lanes
    // idle in one to four waves (5 at 5120 channels: 128 threads, none idle)
    if (ngroups <= 8 && D <= 256 * 8 * 8) {
        const int Di = (int)D, Dg = (int)(D / ngroups), ng = (int)ngroups;
        const int64_t npc = D / 8;
        int best = 0;
        int64_t best_idle = INT64_MAX;
        for (int m : {4, 5, 8}) {
            const int64_t nthr = ((npc + m - 1) / m + 63) / 64 * 64;
            if (nthr > 256) continue;
            const int64_t idle = nthr * m - npc;
            if (idle < best_idle) best_idle = idle, best = m;
        }
        const unsigned nthr = (unsigned)(((npc + best - 1) / best + 63) / 64 * 64);
#define SSD_GN_LAUNCH(M)                                                                               \
    if (d.dtype == 1)                                                                                  \
        k_gated_rmsnorm_reg<bf16, M><<<(unsigned)rows, nthr, 0, st>>>((const bf16 *)y, (const bf16 *)z, \
                                                                    w, (bf16 *)out, Di, Dg, ng, eps);  \
    else                                                                                               \
        k_gated_rmsnorm_reg<float, M><<<(unsigned)rows, nthr, 0, st>>>(                              \
            (const float *)y, (const float *)z, w, (float *)out, Di, Dg, ng, eps);
        if (best == 4) { SSD_GN_LAUNCH(4) }
        else if (best == 5) { SSD_GN_LAUNCH(5) }
        else { SSD_GN_LAUNCH(8) }
#undef SSD_GN_LAUNCH
        return hipGetLastError();
    }
    if (d.dtype == 1)
        k_gated_rmsnorm<bf16><<<(unsigned)rows, 256, 0, st>>>((const bf16 *)y, (const bf16 *)z, w,
                                                              (bf16 *)out, D, D / ngroups,
                                                              (int)ngroups, eps);
    else
        k_gated_rmsnorm<float><<<(unsigned)rows, 256, 0, st>>>((const float *)y, (const float *)z, w,
                                                               (float *)out, D, D / ngroups,
                                                               (int)ngroups, eps);
    return hipGetLastError();
}

}  // namespace ssd
