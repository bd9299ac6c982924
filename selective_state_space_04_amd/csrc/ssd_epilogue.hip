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
// NT: non-temporal accesses, for data that streams through once
template <> struct Vec8<bf16> {
    template <bool NT = false>
    static __device__ __forceinline__ void load(const bf16 *p, float *v) {
        const u32x4 w = NT ? __builtin_nontemporal_load((const u32x4 *)p) : *(const u32x4 *)p;
        const bf16x8 t = as_bf16x8(w);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (float)t[e];
    }
    template <bool NT = false>
    static __device__ __forceinline__ void store(bf16 *p, const float *v) {
        bf16x8 t;
#pragma unroll
        for (int e = 0; e < 8; ++e) t[e] = (bf16)v[e];
        if (NT) __builtin_nontemporal_store(as_u32x4(t), (u32x4 *)p);
        else *(bf16x8 *)p = t;
    }
};
template <> struct Vec8<float> {
    template <bool NT = false>
    static __device__ __forceinline__ void load(const float *p, float *v) {
        const f32x4 a = NT ? __builtin_nontemporal_load((const f32x4 *)p) : *(const f32x4 *)p;
        const f32x4 b = NT ? __builtin_nontemporal_load((const f32x4 *)(p + 4)) : *(const f32x4 *)(p + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            v[e] = a[e];
            v[e + 4] = b[e];
        }
    }
    template <bool NT = false>
    static __device__ __forceinline__ void store(float *p, const float *v) {
        const f32x4 a = f32x4{v[0], v[1], v[2], v[3]}, b = f32x4{v[4], v[5], v[6], v[7]};
        if (NT) {
            __builtin_nontemporal_store(a, (f32x4 *)p);
            __builtin_nontemporal_store(b, (f32x4 *)(p + 4));
        } else {
            *(f32x4 *)p = a;
            *(f32x4 *)(p + 4) = b;
        }
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

// Rows of at most 128 * 8 * MAXP channels and at most 8 groups: one pass.
// 128 threads per row; each keeps g for its (up to MAXP) 8-channel pieces in
// registers, accumulates g^2 per group, and after one fixed-order reduction
// per group scales and stores them, so y and z are read once.
template <typename T, int MAXP>
__global__ __launch_bounds__(128) void k_gated_rmsnorm_reg(const T *y, const T *__restrict__ z,
                                                           const float *__restrict__ w, T *out,
                                                           int D, int Dg, int ngroups, float eps) {
    const int64_t row = blockIdx.x;
    const T *yr = y + row * D;
    const T *zr = z + row * D;
    T *orow = out + row * D;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int npieces = D / 8;
    float g[MAXP][8];
    float ss[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) ss[k] = 0.f;
#pragma unroll
    for (int u = 0; u < MAXP; ++u) {
        const int pc = tid + 128 * u;
        if (pc < npieces) {
            float yv[8], zv[8];
            Vec8<T>::template load<true>(yr + 8 * pc, yv);
            Vec8<T>::template load<true>(zr + 8 * pc, zv);
            float acc = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                g[u][e] = yv[e] * silu(zv[e]);
                acc += g[u][e] * g[u][e];
            }
            const int gi = (8 * pc) / Dg;
#pragma unroll
            for (int k = 0; k < 8; ++k) ss[k] += (k == gi) ? acc : 0.f;
        }
    }
    __shared__ float red[2][8];
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
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 8; ++k)
        scale[k] = k < ngroups ? rsqrtf((red[0][k] + red[1][k]) / (float)Dg + eps) : 0.f;
#pragma unroll
    for (int u = 0; u < MAXP; ++u) {
        const int pc = tid + 128 * u;
        if (pc < npieces) {
            const int gi = (8 * pc) / Dg;
            float sc = 0.f;
#pragma unroll
            for (int k = 0; k < 8; ++k) sc = (k == gi) ? scale[k] : sc;
            const f32x4 w0 = *(const f32x4 *)(w + 8 * pc), w1 = *(const f32x4 *)(w + 8 * pc + 4);
            float o[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] = g[u][e] * sc * (e < 4 ? w0[e] : w1[e - 4]);
            Vec8<T>::template store<true>(orow + 8 * pc, o);
        }
    }
}

hipError_t launch_gated_rmsnorm(const Dims &d, int64_t ngroups, float eps, const void *y,
                                const void *z, const float *w, void *out, hipStream_t st) {
    const int64_t rows = d.b * d.L, D = d.H * d.P;
    if (rows == 0) return hipSuccess;
    if (ngroups <= 8 && D <= 128 * 8 * 8) {
        const int Di = (int)D, Dg = (int)(D / ngroups), ng = (int)ngroups;
        if (d.dtype == 1)
            k_gated_rmsnorm_reg<bf16, 8><<<(unsigned)rows, 128, 0, st>>>(
                (const bf16 *)y, (const bf16 *)z, w, (bf16 *)out, Di, Dg, ng, eps);
        else
            k_gated_rmsnorm_reg<float, 8><<<(unsigned)rows, 128, 0, st>>>(
                (const float *)y, (const float *)z, w, (float *)out, Di, Dg, ng, eps);
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
