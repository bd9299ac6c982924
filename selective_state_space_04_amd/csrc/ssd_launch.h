// Host-side launchers of the SSD kernels (internal to libssd_mi355x.so).
// Shapes are validated by the C-ABI layer before any launcher is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ssd_device.h"

namespace ssd {

struct Dims {
    int64_t b, L, H, P, N, G, Q, nc;
    int dtype;  // 0 = f32, 1 = bf16
};

hipError_t launch_chunk_cumsum(const Dims &d, const void *dt, const float *A, float *cs,
                               hipStream_t st);
// With step-size options: cs from the preprocessed dt and, when sc is given,
// the input scale of every step (same layout as cs).
hipError_t launch_chunk_cumsum_opts(const Dims &d, const void *dt, const float *A,
                                    const DtOpts &o, float *cs, float *sc, hipStream_t st);
hipError_t launch_chunk_cb(const Dims &d, const void *B, const void *C, void *cb, void *cbT,
                           hipStream_t st);
hipError_t launch_chunk_state(const Dims &d, const void *x, const void *B, const float *cs,
                              float *S, bool from_start, hipStream_t st,
                              const float *sc = nullptr);
hipError_t launch_state_passing(const Dims &d, float *S, const float *cs, const float *init,
                                float *fin, hipStream_t st);
hipError_t launch_chunk_scan(const Dims &d, const void *x, const void *C, const void *cb,
                             const float *cs, const float *hprev, const float *D, void *y,
                             hipStream_t st, const float *sc = nullptr);
// Decode: batch * nheads * headdim state rows at most (32-bit row indices).
constexpr int64_t kDecodeMaxRows = ((int64_t)1 << 31) - 4096;
hipError_t launch_decode(const Dims &d, float *state, const void *x, const void *dt,
                         const float *A, const void *B, const void *C, const float *D, void *y,
                         hipStream_t st, const DtOpts *o = nullptr);
// Single-pass forward (ssd_walk.hip): bfloat16, P = 64, N = 128.  The
// preparation writes every 32-step chunk's operands (per group) and decay
// records (per head) into the workspace; the walk reads them.
bool walk_supported(const Dims &d);
struct WalkBytes {
    int64_t ops;  // fragment-ordered C, B^T and causal C B^T of every chunk and group
    int64_t rec;  // decay record of every chunk and head
};
WalkBytes walk_bytes(const Dims &d);
hipError_t launch_walk_prep(const Dims &d, const void *dt, const float *A, const void *B, const void *C,
                            void *ops, float *rec, hipStream_t st, const DtOpts *o = nullptr);
hipError_t launch_walk_main(const Dims &d, const void *x, const void *ops, const float *rec, const float *D,
                            const float *init, void *y, float *fin, hipStream_t st, bool opts);
hipError_t launch_zero_state(const Dims &d, const float *init, float *fin, hipStream_t st);

// Selective (Mamba-1) scan (ssd_scan.hip).  algo 1 = segments (seg steps per
// segment, nseg segments per sequence; S = segment states, sdl = step sums);
// algo 2 = rows (N = 16; S = B and C transposed to float32 [b, G, N, Lp], Lp
// = L rounded up to 16, B first).
struct ScanDims {
    int64_t b, L, Dch, N, G, seg, nseg, Lp;
    int dtype;  // 0 = f32, 1 = bf16
    int algo;
};
hipError_t launch_selective_scan(const ScanDims &d, const void *x, const void *delta,
                                 const float *A, const void *B, const void *C, const float *D,
                                 const void *z, const float *dbias, int softplus,
                                 const float *init, void *y, float *fin, float *S, float *sdl,
                                 hipStream_t st, void *const *marks = nullptr, int nmarks = 0);

// Normalisation after the gate (ssd_epilogue.hip).
hipError_t launch_gated_rmsnorm(const Dims &d, int64_t ngroups, float eps, const void *y,
                                const void *z, const float *w, void *out, hipStream_t st);

// Gradient kernels (ssd_backward.hip).
hipError_t launch_state_passing_rev(const Dims &d, float *S, const float *cs, const float *dfinal,
                                    float *dinit, hipStream_t st);
hipError_t launch_chunk_cumsum64(const Dims &d, const void *dt, const float *A, double *cs,
                                 hipStream_t st);
// bfloat16 chunk backward with its operands in fragment order: when true,
// launch_chunk_bwd reads C, B and C B^T from the arrays launch_bwd_frags
// writes (Gy and Gx in place of cb and cbT, whose workspace slots they take;
// sizes in bwd_frag_bytes) and ignores B, C, cb's row-major form.
bool chunk_bwd_frags(const Dims &d);
struct BwdFragBytes {
    int64_t rows;    // Cf, Bf each
    int64_t blocks;  // Gy, Gx each
    int64_t diag;    // dg
};
BwdFragBytes bwd_frag_bytes(const Dims &d);
hipError_t launch_bwd_frags(const Dims &d, const void *B, const void *C, void *Gy, void *Gx,
                            void *Cf, void *Bf, float *dg, hipStream_t st);
hipError_t launch_chunk_bwd(const Dims &d, const void *x, const void *dy, const void *dt,
                            const float *A, const void *B, const void *C, const void *cb,
                            const void *cbT, const void *Cf, const void *Bf, const float *dg,
                            const float *cs, const double *cs64, const float *Hs, const float *Rs,
                            const float *D, void *dx, void *ddt, float *part, hipStream_t st);
hipError_t launch_group_bwd(const Dims &d, const void *x, const void *dy, const float *cs,
                            const double *cs64, const float *Hs, const float *Rs, float *dcb,
                            float *dcbT, float *dCs, float *dBs, hipStream_t st);
hipError_t launch_group_combine(const Dims &d, const void *B, const void *C, const float *dcb,
                                const float *dcbT, const float *dCs, const float *dBs, void *dB,
                                void *dC, hipStream_t st);
hipError_t launch_head_reduce(const Dims &d, const float *part, float *dA, float *dD,
                              hipStream_t st);

}  // namespace ssd
