// Selective (Mamba-1) scan on gfx950 (Mamba review page, section 3.3: per
// channel d a diagonal A[d, :], h_t = exp(dt_t A) * h_{t-1} + dt_t x_t B_t,
// y_t = C_t . h_t; section 3.4: skip term D x and the output gated by SiLU(z);
// section 3.1: dt = softplus(dt + bias)).
//
// There is no dense contraction here: each (step, channel, state) costs one
// exp and a few fused multiply-adds, so the scan is bound by the vector ALU.
// Two arrangements:
//
// Rows (N = 16, enough channels): a lane owns one (channel, state) pair, so a
// 16-lane row of the wave is one channel and the whole sequence runs in one
// pass.  Per block of 16 steps, lane q of a row holds the step size and input
// of step q (computed once per element by the workgroup, see k_scan_rows);
// the recurrence takes them from that lane with a DPP row broadcast folded
// into its multiplies; each lane keeps its 16 products C_t[n] h_t[n] and an
// LDS transpose hands lane q the 16 terms of step q, which it sums and
// finishes.  B and C are first converted to float32 tiles so a lane reads
// its state's steps in 16-byte loads that together cover whole cache lines.
//
// Segments (other N, or few channels): a lane owns one channel and its N
// states in registers; the sequence is cut into segments so that enough waves
// run at once:
//   k_scan_seg_state  per (b, segment, 64 channels): the segment's end state
//                     from zero, and the sum of its steps
//   k_scan_pass       per (b, channel, n): the state entering every segment,
//                     exp(A sum dt) h + S across segments; the final state
//   k_scan_seg_out    per (b, segment, 64 channels): rescan from the entering
//                     state, writing y
// The 64 channels of a wave lie in one B/C group, so B_t and C_t are the same
// for the whole wave and come through scalar loads.
#include "ssd_device.h"
#include "ssd_launch.h"

namespace ssd {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// N consecutive values of a wave-uniform row (every lane reads the same
// bytes, so the loads go through the scalar unit): fetched raw in 16-byte
// pieces when the row is a whole number of them, converted to float later,
// so a step's rows can be requested one step before they are used.
template <typename T, int N>
struct RawRow {
    static constexpr bool kVec = (N * (int)sizeof(T)) % 16 == 0;
    static constexpr int kPieces = kVec ? N * (int)sizeof(T) / 16 : 1;
    u32x4 w[kPieces];
    float f[kVec ? 1 : N];
    __device__ __forceinline__ void load(const T *p) {
        if constexpr (kVec) {
#pragma unroll
            for (int c = 0; c < kPieces; ++c) w[c] = *(const u32x4 *)(p + c * (16 / (int)sizeof(T)));
        } else {
#pragma unroll
            for (int n = 0; n < N; ++n) f[n] = to_f32(p[n]);
        }
    }
    __device__ __forceinline__ void get(float *v) const {
        if constexpr (kVec) {
#pragma unroll
            for (int c = 0; c < kPieces; ++c) {
                if constexpr (sizeof(T) == 2) {
                    const bf16x8 t = as_bf16x8(w[c]);
#pragma unroll
                    for (int e = 0; e < 8; ++e) v[c * 8 + e] = (float)t[e];
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const uint32_t u = w[c][e];
                        v[c * 4 + e] = __builtin_bit_cast(float, u);
                    }
                }
            }
        } else {
#pragma unroll
            for (int n = 0; n < N; ++n) v[n] = f[n];
        }
    }
};

// 2^v with the hardware exponential (results below 2^-126 flush to zero,
// which for a decay factor is below every other term's rounding).
__device__ __forceinline__ float fast_exp2(float v) { return __builtin_amdgcn_exp2f(v); }

// softplus(v) = max(v, 0) + log1p(exp(-|v|)), with log1p(e) taken as
// log(w) e / (w - 1), w = 1 + e (w - 1 is exact, so the quotient cancels the
// rounding of w; Goldberg, "What every computer scientist should know about
// floating-point arithmetic", theorem 4), and e itself when w rounds to 1.
__device__ __forceinline__ float softplus_f(float v) {
    const float e = fast_exp2(-fabsf(v) * kLog2e);
    const float w = 1.f + e;
    const float wm1 = w - 1.f;
    const float l = wm1 == 0.f ? e : __builtin_amdgcn_logf(w) * kLn2 * (e * __builtin_amdgcn_rcpf(wm1));
    return fmaxf(v, 0.f) + l;
}

// z * sigmoid(z); exp overflows to inf for z below about -88 and the
// reciprocal then gives 0.
__device__ __forceinline__ float silu_f(float z) {
    return z * __builtin_amdgcn_rcpf(1.f + fast_exp2(-z * kLog2e));
}

// y[lane] = v through a buffer resource of `bytes` bytes at a wave-uniform
// base: lanes past the end fall outside the resource and the hardware drops
// their stores, so masked lanes need no branch (and the count of memory
// operations in flight is the same on every path).
template <typename T>
__device__ __forceinline__ void store_lane(T *base, uint32_t bytes, int lane, T v) {
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(base, (short)0, (int)bytes, 0x00020000);
    if constexpr (sizeof(T) == 2)
        __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, v), rs, lane * 2, 0, 0);
    else
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned int, v), rs, lane * 4, 0, 0);
}

__device__ __forceinline__ float step_size(float raw, float bias, int softplus) {
    const float v = raw + bias;
    return softplus ? softplus_f(v) : v;
}

template <typename T, int N>
__global__ __launch_bounds__(64) void k_scan_seg_state(
    const T *__restrict__ x, const T *__restrict__ delta, const float *__restrict__ A,
    const T *__restrict__ B, const float *__restrict__ dbias, int softplus, float *__restrict__ S,
    float *__restrict__ sdl, int64_t L, int Dch, int G, int seg, int nseg) {
    const int lane = threadIdx.x;
    const int d0 = blockIdx.x * 64, d = d0 + lane;
    const int k = blockIdx.y;
    const int64_t b = blockIdx.z;
    const bool valid = d < Dch;
    const int dc = valid ? d : Dch - 1;  // loads stay in bounds; results are masked
    const int g = d0 / (Dch / G);  // the wave's group
    float a2[N], h[N];
#pragma unroll
    for (int n = 0; n < N; ++n) {
        a2[n] = A[(int64_t)dc * N + n] * kLog2e;
        h[n] = 0.f;
    }
    const float bias = dbias ? dbias[dc] : 0.f;
    float sum = 0.f;
    const int64_t t0 = (int64_t)k * seg, t1 = min<int64_t>(t0 + seg, L);
    // step t + 1's loads are issued before step t computes (the index is
    // clamped, so the same loads are in flight on every path)
    const T *xp = x + b * L * Dch + dc, *dp = delta + b * L * Dch + dc;
    const T *Bp = B + (b * L * G + g) * N;
    T nx = xp[t0 * Dch], nd = dp[t0 * Dch];
    RawRow<T, N> nB;
    nB.load(Bp + t0 * G * N);
    for (int64_t t = t0; t < t1; ++t) {
        const float xv = to_f32(nx), dv = to_f32(nd);
        float bv[N];
        nB.get(bv);
        // scalar loads complete out of order, so their only wait is "all":
        // take it here, before the next step's rows are requested
        __builtin_amdgcn_s_waitcnt(kWaitScalar);
        const int64_t tn = min<int64_t>(t + 1, t1 - 1);
        nx = xp[tn * Dch];
        nd = dp[tn * Dch];
        nB.load(Bp + tn * G * N);
        const float dl = valid ? step_size(dv, bias, softplus) : 0.f;
        const float u = dl * xv;
#pragma unroll
        for (int n = 0; n < N; ++n) h[n] = fast_exp2(dl * a2[n]) * h[n] + u * bv[n];
        sum += dl;
    }
    if (valid) {
        float *o = S + (((b * nseg + k) * Dch + d) * (int64_t)N);
#pragma unroll
        for (int n = 0; n < N; n += 4) *(f32x4 *)(o + n) = f32x4{h[n], h[n + 1], h[n + 2], h[n + 3]};
        sdl[(b * nseg + k) * Dch + d] = sum;
    }
}

// In place: on entry S[k] is segment k's end state from zero; on return the
// state entering segment k.
__global__ __launch_bounds__(256) void k_scan_pass(float *__restrict__ S, const float *__restrict__ sdl,
                                                   const float *__restrict__ A, const float *init,
                                                   float *fin, int Dch, int N, int nseg,
                                                   int64_t total) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= total) return;
    const int64_t DN = (int64_t)Dch * N;
    const int64_t b = idx / DN, dn = idx % DN;
    const int d = (int)(dn / N);
    const float a = A[dn];
    float h = init ? init[idx] : 0.f;
    for (int k = 0; k < nseg; ++k) {
        float *sp = S + (b * nseg + k) * DN + dn;
        const float sv = *sp;
        *sp = h;
        h = __expf(a * sdl[(b * nseg + k) * Dch + d]) * h + sv;
    }
    if (fin) fin[idx] = h;
}

template <typename T, int N>
__global__ __launch_bounds__(64) void k_scan_seg_out(
    const T *__restrict__ x, const T *__restrict__ delta, const float *__restrict__ A,
    const T *__restrict__ B, const T *__restrict__ C, const float *__restrict__ D,
    const T *__restrict__ z, const float *__restrict__ dbias, int softplus,
    const float *__restrict__ S, T *__restrict__ y, int64_t L, int Dch, int G, int seg, int nseg) {
    const int lane = threadIdx.x;
    const int d0 = blockIdx.x * 64, d = d0 + lane;
    const int k = blockIdx.y;
    const int64_t b = blockIdx.z;
    const bool valid = d < Dch;
    const int dc = valid ? d : Dch - 1;  // loads stay in bounds; results are masked
    const int g = d0 / (Dch / G);
    float a2[N], h[N];
    const float *hin = S + (((b * nseg + k) * Dch + dc) * (int64_t)N);
#pragma unroll
    for (int n = 0; n < N; ++n) {
        a2[n] = A[(int64_t)dc * N + n] * kLog2e;
        h[n] = hin[n];
    }
    const float Dd = D ? D[dc] : 0.f;
    const float bias = dbias ? dbias[dc] : 0.f;
    const int64_t t0 = (int64_t)k * seg, t1 = min<int64_t>(t0 + seg, L);
    // step t + 1's loads are issued before step t computes (clamped index;
    // without a gate the z load reads x, so every path has the same loads)
    const int64_t rb = b * L * Dch + dc;
    const T *xp = x + rb, *dp = delta + rb, *zp = (z ? z : x) + rb;
    const T *Bp = B + (b * L * G + g) * N, *Cp = C + (b * L * G + g) * N;
    T nx = xp[t0 * Dch], nd = dp[t0 * Dch], nz = zp[t0 * Dch];
    RawRow<T, N> nB, nC;
    nB.load(Bp + t0 * G * N);
    nC.load(Cp + t0 * G * N);
    for (int64_t t = t0; t < t1; ++t) {
        const float xv = to_f32(nx), dv = to_f32(nd), zv = to_f32(nz);
        float bv[N], cv[N];
        nB.get(bv);
        nC.get(cv);
        __builtin_amdgcn_s_waitcnt(kWaitScalar);  // as in k_scan_seg_state
        const int64_t tn = min<int64_t>(t + 1, t1 - 1);
        nx = xp[tn * Dch];
        nd = dp[tn * Dch];
        nz = zp[tn * Dch];
        nB.load(Bp + tn * G * N);
        nC.load(Cp + tn * G * N);
        const float dl = step_size(dv, bias, softplus);
        const float u = dl * xv;
        float acc = 0.f;
#pragma unroll
        for (int n = 0; n < N; ++n) {
            h[n] = fast_exp2(dl * a2[n]) * h[n] + u * bv[n];
            acc += cv[n] * h[n];
        }
        float out = acc + Dd * xv;
        if (z) out *= silu_f(zv);
        store_lane<T>(y + (b * L + t) * Dch + d0, (uint32_t)(Dch - d0) * (uint32_t)sizeof(T), lane,
                      from_f32<T>(out));
    }
}


// ---------------------------------------------------------------- rows path

// B or C [b, L, G, N] (dtype T) -> float32 tiles of 16 steps: for each
// (b, g, tile) four groups of 4 steps, each [N][4]; zero past L.  A lane that
// owns state n reads its 4 steps of a group as one 16-byte load, and the 16
// states of the group are 256 contiguous bytes.
template <typename T>
__global__ __launch_bounds__(256) void k_scan_bc_tile(const T *__restrict__ B, const T *__restrict__ C,
                                                      float *__restrict__ BT, float *__restrict__ CT,
                                                      int64_t L, int64_t ntile, int G, int N, int64_t total) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;  // over [b, G, ntile, 4, N, 4]
    if (idx >= total) return;
    const int e = (int)(idx & 3);
    const int n = (int)((idx >> 2) % N);
    const int64_t r = (idx >> 2) / N;             // ((b * G + g) * ntile + tile) * 4 + k
    const int k = (int)(r & 3);
    const int64_t tile = (r >> 2) % ntile;
    const int64_t bg = (r >> 2) / ntile;
    const int g = (int)(bg % G);
    const int64_t b = bg / G;
    const int64_t t = tile * 16 + k * 4 + e;
    float bv = 0.f, cv = 0.f;
    if (t < L) {
        const int64_t src = ((b * L + t) * G + g) * N + n;
        bv = to_f32(B[src]);
        cv = to_f32(C[src]);
    }
    BT[idx] = bv;
    CT[idx] = cv;
}

// Lane J of each 16-lane row, broadcast to its row (DPP row_newbcast).
template <int J>
__device__ __forceinline__ float row_bcast(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                                 0x150 + J, 0xF, 0xF, false));
}

// Steps J..15 of a block: h = exp(dt A) h + (dt x) B; the term C h of step
// J goes straight to column q of line J of the row's LDS block.
template <int J>
__device__ __forceinline__ void rows_steps(float dl, float u, float a2, const f32x4 *bv, const f32x4 *cv,
                                           float &h, float *col) {
    const float e = fast_exp2(row_bcast<J>(dl) * a2);
    const float ub = __fmul_rn(row_bcast<J>(u), bv[J / 4][J % 4]);
    h = __builtin_fmaf(e, h, ub);
    col[J * 20] = cv[J / 4][J % 4] * h;
    if constexpr (J < 15) rows_steps<J + 1>(dl, u, a2, bv, cv, h, col);
}

// Workgroup index spread so that consecutive logical indices stay on one of
// the 8 XCDs (workgroups are dealt to XCDs in turn); neighbouring channel
// blocks then share that XCD's L2 for the cache lines they split.
__device__ __forceinline__ int64_t xcd_local(int64_t wg, int64_t total) {
    const int64_t per = total / 8, rem = total % 8, x = wg % 8, k = wg / 8;
    return x < rem ? x * (per + 1) + k : rem * (per + 1) + (x - rem) * per + k;
}

constexpr int kRowQS = 20;   // LDS stride between a row's 16 lanes (words)
constexpr int kRowRS = 336;  // LDS stride between rows: 16 * 20 + 16

// One workgroup: 4 waves x 4 rows = 16 channels of one batch row, N = 16.
// Per block of 16 steps, thread i = (step i / 16, channel i % 16) loads that
// element of x, delta and z (16 threads read 32 contiguous bytes), computes
// the step size, the input dt x, the skip term D x and the gate, and hands
// them through LDS to lane q of that channel's row; after the scan the
// row's outputs go back through LDS so the stores are contiguous too.  One
// workgroup barrier per block: the inputs of block k+1 are prepared, and the
// raw values of block k+2 requested, while block k is scanned.  B and C of a
// block are requested at its start; they are shared by every row and stay
// in cache, and the other workgroups on the SIMD cover the wait.  Five
// workgroups per CU (LDS) fill the chip at the Mamba-2.8B layer width.
// Offsets within one batch row are 32-bit (L * channels < 2^31).
template <typename T>
__global__ __launch_bounds__(256) void k_scan_rows(
    const T *__restrict__ x, const T *__restrict__ delta, const float *__restrict__ A,
    const float *__restrict__ BT, const float *__restrict__ CT, const float *__restrict__ D,
    const T *__restrict__ z, const float *__restrict__ dbias, int softplus, const float *init,
    T *__restrict__ y, float *fin, int L, int ntile, int Dch, int G, int nblk) {
    constexpr int N = 16;
    constexpr int IS = 17;  // float4 stride between channels of the input buffer
    constexpr int OS = 17;  // word stride between steps of the output buffer
    __shared__ __attribute__((aligned(16))) float red[4 * 4 * kRowRS];
    __shared__ __attribute__((aligned(16))) f32x4 inb[2][16 * IS];
    __shared__ float outb[2][16 * OS];
    const int wg = (int)xcd_local(blockIdx.x, gridDim.x);
    const int b = wg / nblk;
    const int blk = wg % nblk;
    const int tid = threadIdx.x;
    const int w = tid >> 6, l = tid & 63, r = l >> 4, q = l & 15;
    // scanning lane: channel cs of the block, state q, step q of each block
    const int cs = w * 4 + r;
    const int d = blk * 16 + cs;
    const bool valid = d < Dch;
    const int dc = valid ? d : Dch - 1;
    const int g = (blk * 16) / (Dch / G);        // 16 channels never straddle a group
    const float a2 = A[dc * N + q] * kLog2e;
    float h = (init && valid) ? init[((int64_t)b * Dch + d) * N + q] : 0.f;
    const f32x4 *bt = (const f32x4 *)(BT + ((int64_t)b * G + g) * ntile * 16 * N) + q;
    const f32x4 *ct = (const f32x4 *)(CT + ((int64_t)b * G + g) * ntile * 16 * N) + q;
    float *row = red + cs * kRowRS;
    // loading thread: step pt of the block, channel pc
    const int pt = tid >> 4, pc = tid & 15;
    const int pd = blk * 16 + pc;
    const bool pvalid = pd < Dch;
    const int pdc = pvalid ? pd : Dch - 1;       // loads stay in bounds; results are masked
    const float bias = dbias ? dbias[pdc] : 0.f;
    const float Dd = D ? D[pdc] : 0.f;
    const int64_t rowbase = (int64_t)b * L * Dch;
    const bool has_z = z != nullptr;
    // without a gate, z's load reads x again (an unconditional load keeps the
    // count of loads in flight the same on every path)
    const T *xb = x + rowbase, *db = delta + rowbase, *zb = (has_z ? z : x) + rowbase;
    T *yb = y + rowbase;
    T rx = T(0), rd = T(0), rz = T(0);
    auto load_raw = [&](int t0) {
        const int off = min(t0 + pt, L - 1) * Dch + pdc;
        rx = xb[off];
        rd = db[off];
        rz = zb[off];
    };
    // step size, input, skip and gate of (t0 + pt, pc) into inb[buf]
    auto prepare = [&](int t0, int buf) {
        const float xv = to_f32(rx);
        float dl = step_size(to_f32(rd), bias, softplus);
        dl = (t0 + pt < L) ? dl : 0.f;           // padded steps leave h unchanged
        const float gate = has_z ? silu_f(to_f32(rz)) : 1.f;
        inb[buf][pc * IS + pt] = f32x4{dl, dl * xv, Dd * xv, gate};
    };
    load_raw(0);
    prepare(0, 0);
    if (ntile > 1) load_raw(16);
    lds_barrier();
    for (int tile = 0; tile < ntile; ++tile) {
        const int buf = tile & 1;
        const int t0 = tile * 16;
        f32x4 bv[4], cv[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            bv[k] = bt[(tile * 4 + k) * N];
            cv[k] = ct[(tile * 4 + k) * N];
        }
        if (tile + 1 < ntile) prepare(t0 + 16, buf ^ 1);
        load_raw(t0 + 32);  // clamped in range; issued on every path so the wait counts stay exact
        const f32x4 in = inb[buf][cs * IS + q];
        // transpose through LDS: lane q scatters its 16 terms (term j to
        // column q of line j), then reads line q, the 16 terms of step q (the
        // row's lanes only talk to each other, so the wave's in-order LDS
        // queue is the only ordering needed)
        __builtin_amdgcn_wave_barrier();
        rows_steps<0>(in[0], in[1], a2, bv, cv, h, row + q);
        __builtin_amdgcn_wave_barrier();
        f32x4 tv[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) tv[k] = *(const f32x4 *)(row + q * kRowQS + 4 * k);
        float acc = 0.f;
#pragma unroll
        for (int k = 0; k < 4; ++k) acc += (tv[k][0] + tv[k][1]) + (tv[k][2] + tv[k][3]);
        outb[buf][q * OS + cs] = (acc + in[2]) * in[3];
        lds_barrier();
        if (pvalid && t0 + pt < L) yb[(t0 + pt) * Dch + pd] = from_f32<T>(outb[buf][pt * OS + pc]);
    }
    if (fin && valid) fin[((int64_t)b * Dch + d) * N + q] = h;
}

#define SSD_SCAN_DISPATCH_N(N_, ...)                                              \
    switch (N_) {                                                                 \
    case 4: { constexpr int NN = 4; __VA_ARGS__; } break;                         \
    case 8: { constexpr int NN = 8; __VA_ARGS__; } break;                         \
    case 16: { constexpr int NN = 16; __VA_ARGS__; } break;                       \
    case 32: { constexpr int NN = 32; __VA_ARGS__; } break;                       \
    case 64: { constexpr int NN = 64; __VA_ARGS__; } break;                       \
    default: return hipErrorInvalidValue;                                         \
    }

hipError_t launch_selective_scan(const ScanDims &d, const void *x, const void *delta,
                                 const float *A, const void *B, const void *C, const float *D,
                                 const void *z, const float *dbias, int softplus,
                                 const float *init, void *y, float *fin, float *S, float *sdl,
                                 hipStream_t st, void *const *marks, int nmarks) {
    // marks[k] (when given) is recorded on st before the first launch and
    // after each of the three; with nothing to launch they are recorded at once
    int km = 0;
    auto mark = [&]() -> hipError_t {
        return (marks && km < nmarks) ? hipEventRecord((hipEvent_t)marks[km++], st) : hipSuccess;
    };
    auto mark_rest = [&]() -> hipError_t {
        hipError_t e = hipSuccess;
        while (marks && km < nmarks && e == hipSuccess) e = mark();
        return e;
    };
    hipError_t e;
    if ((e = mark()) != hipSuccess) return e;
    if (d.b == 0) return mark_rest();
    if (d.L == 0) {
        if (fin) {
            const int64_t n = d.b * d.Dch * d.N;
            Dims dd{};
            dd.b = 1; dd.H = 1; dd.P = 1; dd.N = n;  // a flat copy of n floats
            if ((e = launch_zero_state(dd, init, fin, st)) != hipSuccess) return e;
        }
        return mark_rest();
    }
    if (d.algo == 2) {
        const int64_t ntile = d.Lp / 16;
        float *BT = S, *CT = S + d.b * d.G * d.N * d.Lp;
        const int64_t total = d.b * d.G * d.N * d.Lp;
        const unsigned tb = (unsigned)((total + 255) / 256);
        if (d.dtype == 1)
            k_scan_bc_tile<bf16><<<tb, 256, 0, st>>>((const bf16 *)B, (const bf16 *)C, BT, CT, d.L, ntile,
                                                     (int)d.G, (int)d.N, total);
        else
            k_scan_bc_tile<float><<<tb, 256, 0, st>>>((const float *)B, (const float *)C, BT, CT, d.L, ntile,
                                                      (int)d.G, (int)d.N, total);
        if ((e = hipGetLastError()) != hipSuccess || (e = mark()) != hipSuccess) return e;
        const int nblk = (int)((d.Dch + 15) / 16);
        const unsigned grid = (unsigned)(d.b * nblk);
        if (d.dtype == 1)
            k_scan_rows<bf16><<<grid, 256, 0, st>>>((const bf16 *)x, (const bf16 *)delta, A, BT, CT, D,
                                                    (const bf16 *)z, dbias, softplus, init, (bf16 *)y, fin,
                                                    (int)d.L, (int)ntile, (int)d.Dch, (int)d.G, nblk);
        else
            k_scan_rows<float><<<grid, 256, 0, st>>>((const float *)x, (const float *)delta, A, BT, CT, D,
                                                     (const float *)z, dbias, softplus, init, (float *)y,
                                                     fin, (int)d.L, (int)ntile, (int)d.Dch, (int)d.G, nblk);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        return mark_rest();
    }
    const dim3 grid((unsigned)((d.Dch + 63) / 64), (unsigned)d.nseg, (unsigned)d.b);
    const int Dch = (int)d.Dch, G = (int)d.G, seg = (int)d.seg, nseg = (int)d.nseg;
    SSD_SCAN_DISPATCH_N(d.N, {
        if (d.dtype == 1)
            k_scan_seg_state<bf16, NN><<<grid, 64, 0, st>>>((const bf16 *)x, (const bf16 *)delta, A,
                                                           (const bf16 *)B, dbias, softplus, S, sdl,
                                                           d.L, Dch, G, seg, nseg);
        else
            k_scan_seg_state<float, NN><<<grid, 64, 0, st>>>((const float *)x, (const float *)delta, A,
                                                            (const float *)B, dbias, softplus, S, sdl,
                                                            d.L, Dch, G, seg, nseg);
    });
    if ((e = hipGetLastError()) != hipSuccess || (e = mark()) != hipSuccess) return e;
    const int64_t total = d.b * d.Dch * d.N;
    k_scan_pass<<<(unsigned)((total + 255) / 256), 256, 0, st>>>(S, sdl, A, init, fin, Dch, (int)d.N,
                                                                 nseg, total);
    if ((e = hipGetLastError()) != hipSuccess || (e = mark()) != hipSuccess) return e;
    SSD_SCAN_DISPATCH_N(d.N, {
        if (d.dtype == 1)
            k_scan_seg_out<bf16, NN><<<grid, 64, 0, st>>>((const bf16 *)x, (const bf16 *)delta, A,
                                                         (const bf16 *)B, (const bf16 *)C, D,
                                                         (const bf16 *)z, dbias, softplus, S,
                                                         (bf16 *)y, d.L, Dch, G, seg, nseg);
        else
            k_scan_seg_out<float, NN><<<grid, 64, 0, st>>>((const float *)x, (const float *)delta, A,
                                                          (const float *)B, (const float *)C, D,
                                                          (const float *)z, dbias, softplus, S,
                                                          (float *)y, d.L, Dch, G, seg, nseg);
    });
    if ((e = hipGetLastError()) != hipSuccess) return e;
    return mark_rest();
}

}  // namespace ssd
