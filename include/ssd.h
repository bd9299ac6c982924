/*
 * ssd.h -- C ABI of the MI355X (gfx950) SSD layer library, libssd_mi355x.so.
 *
 * The SSD layer ("state space dual", the Mamba-2 core; docsaid.org review
 * "Mamba-2", sections "SSM を一つの行列として書く" and "A を一つの数に簡略化する")
 * computes, for every batch row b and head h (group g = h / (H / G)):
 *
 *   a_t    = exp(dt[b,t,h] * A[h])
 *   h_t    = a_t * h_{t-1} + x[b,t,h,:] (outer) B[b,t,g,:]      state [P, N]
 *   y[b,t,h,:] = h_t C[b,t,g,:] + D[h] * x[b,t,h,:]
 *
 * with h_{-1} = init_state (zeros when NULL).  ssd_forward evaluates it with
 * the chunked algorithm (same review, section "2つのルートを半分ずつ"; SSD
 * summary page, section "チャンク化アルゴリズム": the masked attention form
 * inside blocks of `chunk` steps, the recurrence across blocks); the result
 * does not depend on `chunk` except through rounding.  ssd_decode_step is
 * one step of the recurrence on a carried state (review, section
 * "4つのトークンで計算してみる": the recurrent route keeps a constant-size
 * state and suits generation).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Pointers.  Every array pointer is DEVICE memory owned by the caller; the
 *   library never allocates, frees or retains them.  Scratch memory comes in
 *   through `workspace`.  All arrays are dense, row-major and contiguous:
 *     x, y  [batch, seqlen, nheads, headdim]     dtype
 *     dt    [batch, seqlen, nheads]              dtype
 *     B, C  [batch, seqlen, ngroups, dstate]     dtype
 *     A, D  [nheads]                              float32
 *     init_state, final_state, state  [batch, nheads, headdim, dstate]  float32
 *   Decode uses the same layouts with seqlen = 1 (x, y [batch, nheads,
 *   headdim]; dt [batch, nheads]; B, C [batch, ngroups, dstate]).
 *   `dtype` (SSD_F32 or SSD_BF16) is the type of x, dt, B, C and y; states,
 *   A and D are always float32.  Arrays must be 16-byte aligned and the
 *   workspace 256-byte aligned.
 * Streams.  `stream` is a hipStream_t passed as void* (NULL = the default
 *   stream).  Calls only enqueue work on it; they never synchronise.
 * Errors.  Argument errors are detected on the host before anything is
 *   enqueued, and then nothing is written.  A failed launch returns
 *   SSD_ERR_HIP.  Input VALUES are not checked: NaN/Inf propagate, and A > 0
 *   or dt < 0 are evaluated as the defined recurrence (they may overflow).
 * Aliasing.  y must not overlap any input.  final_state may be the same
 *   array as init_state (in-place carry) but must not partially overlap it
 *   or overlap anything else.
 * Supported shapes.  headdim in {16, 32, 64, 128}; dstate in
 *   {16, 32, 64, 128, 256}; chunk a multiple of 16 in [16, 256]; nheads a
 *   multiple of ngroups; batch, seqlen >= 0 (seqlen may be any length: the
 *   last chunk may be short).  Others return SSD_ERR_UNSUPPORTED.
 */
#ifndef SSD_MI355X_H
#define SSD_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SSD_OK = 0,
    SSD_ERR_NULL = 1,        /* a required pointer is NULL */
    SSD_ERR_SHAPE = 2,       /* a negative or inconsistent size */
    SSD_ERR_DTYPE = 3,       /* dtype is not SSD_F32 / SSD_BF16 */
    SSD_ERR_ALIGN = 4,       /* a pointer is not 16-byte (workspace: 256-byte) aligned */
    SSD_ERR_WORKSPACE = 5,   /* workspace too small or NULL when needed */
    SSD_ERR_UNSUPPORTED = 6, /* headdim / dstate / chunk outside the compiled set */
    SSD_ERR_HIP = 7,         /* a HIP call or kernel launch failed */
    SSD_ERR_ALIAS = 8        /* an output overlaps an input it must not overlap */
} ssd_status;

typedef enum { SSD_F32 = 0, SSD_BF16 = 1 } ssd_dtype;

typedef struct {
    int64_t batch;    /* b */
    int64_t seqlen;   /* L (ignored by decode) */
    int64_t nheads;   /* H */
    int64_t headdim;  /* P */
    int64_t dstate;   /* N */
    int64_t ngroups;  /* G: heads h in [k*H/G, (k+1)*H/G) share B, C group k */
    int64_t chunk;    /* Q: block length of the chunked algorithm (ignored by decode) */
    int32_t dtype;    /* ssd_dtype of x, dt, B, C, y */
} ssd_dims;

/* Text for a status code (static storage; never NULL). */
const char *ssd_status_string(ssd_status s);

/* Text of the HIP error behind the calling thread's last SSD_ERR_HIP
 * (static storage; "no error" when there was none). */
const char *ssd_last_hip_error(void);

/* Bytes of workspace ssd_forward / ssd_forward_staged need for these dims
 * (0 for invalid dims).  Pure host computation. */
size_t ssd_forward_workspace_bytes(const ssd_dims *dims);

/*
 * Layer forward over a whole sequence, chunked algorithm (review page,
 * section "2つのルートを半分ずつ").
 *   D           nullable: treated as zeros (the per-head skip term).
 *   init_state  nullable: zeros.
 *   final_state nullable: not written.  Receives h_{L-1}.
 *   workspace   device scratch of at least ssd_forward_workspace_bytes(dims);
 *               its contents on entry are ignored.
 * y receives the outputs in dtype (bfloat16 rounded to nearest even).
 */
ssd_status ssd_forward(const ssd_dims *dims, const void *x, const void *dt, const float *A,
                       const void *B, const void *C, const float *D, const float *init_state,
                       void *y, float *final_state, void *workspace, size_t workspace_bytes,
                       void *stream);

/* Same contract and result as ssd_forward, computed by running the five step
 * kernels below one after another with their intermediates in `workspace`
 * (the unfused reference arrangement of the chunked algorithm). */
ssd_status ssd_forward_staged(const ssd_dims *dims, const void *x, const void *dt,
                              const float *A, const void *B, const void *C, const float *D,
                              const float *init_state, void *y, float *final_state,
                              void *workspace, size_t workspace_bytes, void *stream);

/*
 * The single-pass arrangement ssd_forward uses for bfloat16 inputs with
 * headdim 64 and dstate 128 (any chunk; other shapes use the staged one).
 * One workgroup per (batch, head) walks the whole sequence in 32-step chunks
 * and keeps the state in its registers: inside each chunk the masked
 * attention form, across chunks the recurrence on the carried state (review
 * page, section "2つのルートを半分ずつ": only the end-of-block state passes
 * from block to block).  x is read and y written once, and no state goes
 * through memory.  The chunked algorithm gives the same result for every
 * chunk length (up to rounding), so this route ignores `chunk`.
 * ssd_forward is exactly ssd_forward_prep followed by ssd_forward_main on
 * the same stream and workspace; they are exposed so each launch can be
 * timed on its own.
 *   ssd_forward_prep: for every 32-step chunk, the C, B^T and causal C B^T
 *                     operand tiles of each group and the decay prefix of
 *                     each head (from dt and A) into the workspace.
 *   ssd_forward_main: everything else.  Must follow ssd_forward_prep on the
 *                     same workspace and the same dt, A, B, C, with no other
 *                     use of the workspace in between; its dt, A, B, C
 *                     arguments are validated but not read.
 * Both return SSD_ERR_UNSUPPORTED for shapes outside the single-pass set.
 * ssd_forward_is_single_pass tells whether ssd_forward takes this route. */
int ssd_forward_is_single_pass(const ssd_dims *dims);
ssd_status ssd_forward_prep(const ssd_dims *dims, const void *dt, const float *A, const void *B,
                            const void *C, void *workspace, size_t workspace_bytes, void *stream);
ssd_status ssd_forward_main(const ssd_dims *dims, const void *x, const void *dt, const float *A,
                            const void *B, const void *C, const float *D, const float *init_state,
                            void *y, float *final_state, void *workspace, size_t workspace_bytes,
                            void *stream);

/*
 * ssd_forward for callers that cannot allocate: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  Same contract and
 * result as ssd_forward except that there is no workspace argument: the
 * workspace is a device array of SSD_NOALLOC_WORKSPACE_BYTES inside the
 * library, one per GPU, held from the library's load to the end of the
 * process.  The entry point makes no allocation (no hipMalloc, hipFree or
 * allocating library call); the first call on a device looks up the array's
 * address there (hipGetSymbolAddress, SSD_ERR_HIP if that fails).
 *   Dims whose ssd_forward_workspace_bytes exceeds SSD_NOALLOC_WORKSPACE_BYTES
 *   return SSD_ERR_WORKSPACE before any HIP call (as invalid dims return
 *   their own status).  The array's contents on entry are ignored, as
 *   ssd_forward ignores its workspace's.
 *   All calls on one GPU share its array: calls that overlap in time on one
 *   GPU (on different streams, or from different host threads without
 *   ordering) race on it and must not be made.
 */
#define SSD_NOALLOC_WORKSPACE_BYTES ((size_t)32 << 20)
ssd_status ssd_forward_noalloc(const ssd_dims *dims, const void *x, const void *dt, const float *A,
                               const void *B, const void *C, const float *D, const float *init_state,
                               void *y, float *final_state, void *stream);

/*
 * Step-size preprocessing and input scaling, the neighbours of the core in a
 * Mamba layer, applied inside the kernels.  For every step and head:
 *   dt_eff = softplus(dt + dt_bias)   if dt_softplus  (Mamba review page,
 *            dt + dt_bias             otherwise        section 3.1: the step
 *                                                      size is a softplus of a
 *                                                      linear map, dt_bias its bias)
 *   dt_eff = min(max(dt_eff, dt_min), dt_max)   when dt_max > dt_min
 *   a_t    = exp(dt_eff A_h);   the state update adds s x B^T with
 *   s = 1                          SSD_SCALE_NONE (the SSD pages' +B x)
 *   s = dt_eff                     SSD_SCALE_EULER (Mamba review, section 3.3)
 *   s = (exp(dt_eff A_h) - 1)/A_h  SSD_SCALE_ZOH (Mamba review, section 2.2;
 *                                  guide page, equation (2); dt_eff if A_h = 0)
 * The skip term stays D x on the raw x.  dt_bias: [nheads] float32 device
 * array, nullable (zero bias), 16-byte aligned, must not overlap an output.
 * An unknown input_scale returns SSD_ERR_UNSUPPORTED.  A NULL options
 * pointer, or all fields zero, is the plain map of ssd_forward.
 */
typedef enum { SSD_SCALE_NONE = 0, SSD_SCALE_EULER = 1, SSD_SCALE_ZOH = 2 } ssd_input_scale;
typedef struct {
    const float *dt_bias;  /* [nheads] or NULL */
    int32_t dt_softplus;   /* nonzero: softplus(dt + dt_bias) */
    float dt_min, dt_max;  /* clamp when dt_max > dt_min */
    int32_t input_scale;   /* ssd_input_scale */
} ssd_dt_options;

/* ssd_forward / ssd_forward_staged / ssd_decode_step with step-size options
 * (same contracts otherwise; the same workspace size).  The single-pass
 * arrangement takes the options in its own kernel variant. */
ssd_status ssd_forward_ex(const ssd_dims *dims, const ssd_dt_options *opts, const void *x,
                          const void *dt, const float *A, const void *B, const void *C,
                          const float *D, const float *init_state, void *y, float *final_state,
                          void *workspace, size_t workspace_bytes, void *stream);
ssd_status ssd_forward_staged_ex(const ssd_dims *dims, const ssd_dt_options *opts, const void *x,
                                 const void *dt, const float *A, const void *B, const void *C,
                                 const float *D, const float *init_state, void *y,
                                 float *final_state, void *workspace, size_t workspace_bytes,
                                 void *stream);
ssd_status ssd_decode_step_ex(const ssd_dims *dims, const ssd_dt_options *opts, float *state,
                              const void *x, const void *dt, const float *A, const void *B,
                              const void *C, const float *D, void *y, void *stream);

/*
 * One recurrent step for `batch` sequences (review page, section
 * "4つのトークンで計算してみる").  `state` [batch, H, P, N] float32 is read and
 * overwritten in place with a_t * state + x B^T; y [batch, H, P] receives
 * state C + D x.  dims->seqlen and dims->chunk are ignored.  D nullable.
 * batch * H * P must stay below 2^31 - 4096 (else SSD_ERR_UNSUPPORTED).
 */
ssd_status ssd_decode_step(const ssd_dims *dims, float *state, const void *x, const void *dt,
                           const float *A, const void *B, const void *C, const float *D,
                           void *y, void *stream);

/* ------------------------------------------------------------------------
 * Selective scan (the Mamba-1 scan; Mamba review page, section 3.3): per
 * batch row b and channel d, with a diagonal state matrix A[d, :] of N
 * entries and group g = d / (channels / ngroups),
 *   dt  = delta[b,t,d] + delta_bias[d];  dt = softplus(dt) if delta_softplus
 *         (section 3.1: the step size is a softplus of a linear map)
 *   h_t[n] = exp(dt A[d,n]) h_{t-1}[n] + dt x[b,t,d] B[b,t,g,n]
 *   y[b,t,d] = (sum_n C[b,t,g,n] h_t[n] + D[d] x[b,t,d]) * silu(z[b,t,d])
 *         (section 3.4: skip term D and the gate branch; no gate when z is
 *         NULL)
 * with h_{-1} = init_state (zeros when NULL); final_state receives h_{L-1}.
 * Layouts: x, delta, z, y [batch, seqlen, channels] in dtype; A [channels,
 * dstate] float32; B, C [batch, seqlen, ngroups, dstate] in dtype; D,
 * delta_bias [channels] float32; states [batch, channels, dstate] float32.
 * Nullable: D, z, delta_bias, init_state, final_state.  dstate in {4, 8, 16,
 * 32, 64}; channels a multiple of ngroups, and (channels / ngroups) a
 * multiple of 64 when ngroups > 1 (else SSD_ERR_UNSUPPORTED).  y must not
 * overlap an input or final_state; final_state may be init_state itself.
 * Workspace of ssd_selective_scan_workspace_bytes(dims) bytes, 256-byte
 * aligned (segment end states and step sums).  Same stream and error rules
 * as the layer entry points.
 * ---------------------------------------------------------------------- */
typedef struct {
    int64_t batch, seqlen, channels, dstate, ngroups;
    int32_t dtype;  /* ssd_dtype of x, delta, z, B, C, y */
    int32_t algo;   /* 0: default (segments); 1: segments (any dstate):
                       segment end states, state passing, rescan with
                       output; 2: rows (dstate 16, (seqlen + 16) * channels
                       below 2^31, else SSD_ERR_UNSUPPORTED): one pass with
                       a lane per (channel, state).  Both give the same
                       results up to rounding; the workspace size depends
                       on the choice. */
} ssd_scan_dims;
size_t ssd_selective_scan_workspace_bytes(const ssd_scan_dims *dims);
/* The arrangement a call with these dims runs: 1 (segments: three launches,
 * segment states, state passing, output) or 2 (rows: two launches, the
 * B/C transpose and the scan); minus the ssd_status when dims are invalid. */
int32_t ssd_selective_scan_algo(const ssd_scan_dims *dims);
ssd_status ssd_selective_scan(const ssd_scan_dims *dims, const void *x, const void *delta,
                              const float *A, const void *B, const void *C, const float *D,
                              const void *z, const float *delta_bias, int32_t delta_softplus,
                              const float *init_state, void *y, float *final_state,
                              void *workspace, size_t workspace_bytes, void *stream);
/* The same scan with timing marks: events[0] is recorded on the stream
 * before the first launch and events[k] after launch k (segments: the
 * segment-state, state-passing and output launches; rows: the B/C transpose
 * and the scan), as hipEvent_t handles created by the caller, who reads them
 * with hipEventElapsedTime.  Only the first n_events
 * are recorded; where a launch is skipped (empty batch or sequence) its
 * marks are recorded at once.  SSD_ERR_NULL when n_events > 0 and events is
 * NULL, or n_events < 0. */
ssd_status ssd_selective_scan_timed(const ssd_scan_dims *dims, const void *x, const void *delta,
                                    const float *A, const void *B, const void *C, const float *D,
                                    const void *z, const float *delta_bias, int32_t delta_softplus,
                                    const float *init_state, void *y, float *final_state,
                                    void *workspace, size_t workspace_bytes, void *stream,
                                    void *const *events, int32_t n_events);
ssd_status ssd_validate_selective_scan(const ssd_scan_dims *dims, const void *x, const void *delta,
                                       const float *A, const void *B, const void *C,
                                       const float *D, const void *z, const float *delta_bias,
                                       const float *init_state, const void *y,
                                       const float *final_state, const void *workspace,
                                       size_t workspace_bytes);

/* ------------------------------------------------------------------------
 * Normalisation after the gate (review page, section "Mamba-2 ブロック": one
 * normalisation layer after the SSM output is multiplied by the gate, before
 * the output projection; Mamba review page, section 3.4: the gate is SiLU of a
 * second projection z).  The kind of normalisation is not stated; this is
 * the root-mean-square one.  For every token (b, t), over its H * P channels
 * c = h * P + p split into norm_groups equal contiguous groups:
 *   g_c   = y_c * z_c / (1 + exp(-z_c))
 *   out_c = g_c / sqrt(mean over c's group of g^2 + eps) * weight[c]
 * y, z, out [batch, seqlen, nheads, headdim] in dtype (dims->dstate, ngroups
 * and chunk are checked as for the forward but otherwise unused); weight
 * [nheads * headdim] float32.  out may be y itself (in place) but must not
 * otherwise overlap y, z or weight.  (H * P / norm_groups) must be a
 * multiple of 8 and eps >= 0 (else SSD_ERR_SHAPE).
 * ---------------------------------------------------------------------- */
ssd_status ssd_gated_rmsnorm(const ssd_dims *dims, int64_t norm_groups, float eps, const void *y,
                             const void *z, const float *weight, void *out, void *stream);

/* ------------------------------------------------------------------------
 * Gradient of the layer (reverse-mode differentiation of the map that
 * ssd_forward evaluates; the pages define the forward map, in the review
 * page's sections "SSM を一つの行列として書く" and "2つのルートを半分ずつ", and the
 * gradient is its chain rule, organised by the same chunks).  With
 *   Loss = sum(dy * y) + sum(dfinal_state * final_state)
 * for the y and final_state that ssd_forward returns on the same inputs,
 * it writes
 *   dx  [batch, L, H, P]  dtype     dLoss/dx
 *   ddt [batch, L, H]     dtype     dLoss/ddt
 *   dA  [H]               float32   dLoss/dA (summed over batch and steps)
 *   dB, dC [batch, L, G, N] dtype   dLoss/dB, dLoss/dC (summed over the
 *                                   heads of each group)
 *   dD  [H]               float32   dLoss/dD = sum of dy . x per head
 *   dinit_state [batch, H, P, N] float32  dLoss/dinit_state
 * Inputs are those of ssd_forward plus dy [batch, L, H, P] (dtype) and
 * dfinal_state [batch, H, P, N] (float32).  Nullable: D (zeros),
 * init_state (zeros), dfinal_state (zeros), dD and dinit_state (not
 * written).  Every output must not overlap any input, another output or
 * the workspace.  The forward is recomputed inside (nothing is kept from a
 * forward call); the gradients do not depend on `chunk` except through
 * rounding.  Gradients in dtype are rounded to nearest even from float32
 * accumulators.  Same shape support, alignment, stream and error rules as
 * ssd_forward; argument errors write nothing.  For batch = 0 or L = 0, dA
 * and dD are zero and dinit_state = dfinal_state.
 * ssd_backward_workspace_bytes: bytes of workspace needed (0 for invalid
 * dims; pure host computation).
 */
size_t ssd_backward_workspace_bytes(const ssd_dims *dims);
ssd_status ssd_backward(const ssd_dims *dims, const void *x, const void *dt, const float *A,
                        const void *B, const void *C, const float *D, const float *init_state,
                        const void *dy, const float *dfinal_state, void *dx, void *ddt, float *dA,
                        void *dB, void *dC, float *dD, float *dinit_state, void *workspace,
                        size_t workspace_bytes, void *stream);

/* Timing hook for ssd_backward: the same call and result, and in addition
 * hipEventRecord(events[0]) on `stream` before the first kernel launch and
 * hipEventRecord(events[i + 1]) after launch i, so the caller can time each
 * launch with hipEventElapsedTime.  events: nevents hipEvent_t handles
 * created by the caller (not NULL, not owned); nevents must be
 * ssd_backward_launch_count(dims) + 1 (else SSD_ERR_SHAPE).
 * ssd_backward_launch_count: number of launch slots for these dims (0 for
 * invalid dims); ssd_backward_launch_name(dims, i): the kernel name of slot i
 * (static storage; NULL out of range).  A slot that launches nothing for
 * these dims (the float64 decay prefix, which only float32 inputs use) has
 * an empty interval. */
int ssd_backward_launch_count(const ssd_dims *dims);
const char *ssd_backward_launch_name(const ssd_dims *dims, int i);
ssd_status ssd_backward_timed(const ssd_dims *dims, const void *x, const void *dt, const float *A,
                              const void *B, const void *C, const float *D,
                              const float *init_state, const void *dy, const float *dfinal_state,
                              void *dx, void *ddt, float *dA, void *dB, void *dC, float *dD,
                              float *dinit_state, void *workspace, size_t workspace_bytes,
                              void *stream, void *const *events, int nevents);

/* ------------------------------------------------------------------------
 * The steps of the chunked algorithm, one entry point each.  nc =
 * ceil(seqlen / chunk); chunk c covers steps [c*chunk, min((c+1)*chunk, L)).
 * Intermediates are float32 unless stated.
 * ---------------------------------------------------------------------- */

/* Decay prefix (review page, section "A を一つの数に簡略化する": the mask
 * entries are products of per-step decays, so their logarithms are
 * differences of a running sum).  cs [batch, H, nc, chunk]:
 *   cs[b,h,c,i] = sum_{k = c*chunk .. c*chunk+i} dt[b,k,h] * A[h]
 * computed by a log-depth wavefront scan in float32.  Entries past the end of
 * a short last chunk repeat its last valid value. */
ssd_status ssd_chunk_cumsum(const ssd_dims *dims, const void *dt, const float *A, float *cs,
                            void *stream);

/* C B^T inside each chunk (review page, section "A を一つの数に簡略化する":
 * M = L o (C B^T); the same matrix for every head of a group).
 * cb [batch, nc, G, chunk, chunk] in dtype:  cb[b,c,g,i,j] = C_{s+i} . B_{s+j}.
 * Only 16 x 16 tiles on or below the diagonal are written (rows/columns past
 * the sequence end are zero); tiles above the diagonal are left untouched. */
ssd_status ssd_chunk_cb(const ssd_dims *dims, const void *B, const void *C, void *cb,
                        void *stream);

/* Each chunk's own end state, started from zero (review page, section
 * "2つのルートを半分ずつ": the blocks below the diagonal are low rank and are
 * carried as states).  states [batch, nc, H, P, N] float32:
 *   S[b,c,h] = sum_j exp(cs_e - cs_j) x_{s+j} (outer) B_{s+j}, e = last step of c. */
ssd_status ssd_chunk_state(const ssd_dims *dims, const void *x, const void *B, const float *cs,
                           float *states, void *stream);

/* Inter-chunk recurrence (state-space guide page, equation (3): affine maps
 * compose).  In place on `states`: on entry S[b,c,h], on return the state
 * entering chunk c, hprev[c] (hprev[0] = init or 0; hprev[c+1] =
 * exp(cs_e(c)) hprev[c] + S[c]).  final_state (nullable) receives the state
 * after the last chunk; it may alias init_state. */
ssd_status ssd_state_passing(const ssd_dims *dims, float *states, const float *cs,
                             const float *init_state, float *final_state, void *stream);

/* Intra-chunk masked product plus output combine (SSD summary page,
 * section "チャンク化アルゴリズム": per block (L o Q K^T) V, then the carried
 * state's contribution is added):
 *   y_{s+i} = sum_{j<=i} exp(cs_i - cs_j) cb[i,j] x_{s+j}
 *             + exp(cs_i) hprev[c] C_{s+i} + D x_{s+i}.
 * hprev nullable (zeros: y is then the intra-chunk part plus D x). D nullable. */
ssd_status ssd_chunk_scan(const ssd_dims *dims, const void *x, const void *C, const void *cb,
                          const float *cs, const float *hprev, const float *D, void *y,
                          void *stream);

/* ------------------------------------------------------------------------
 * Host-only argument checks (no HIP call; usable without a GPU).  They
 * return exactly the status the corresponding entry point would return
 * before enqueuing anything.
 * ---------------------------------------------------------------------- */
ssd_status ssd_validate_forward(const ssd_dims *dims, const void *x, const void *dt,
                                const float *A, const void *B, const void *C, const float *D,
                                const float *init_state, const void *y,
                                const float *final_state, const void *workspace,
                                size_t workspace_bytes);
ssd_status ssd_validate_decode(const ssd_dims *dims, const float *state, const void *x,
                               const void *dt, const float *A, const void *B, const void *C,
                               const float *D, const void *y);
ssd_status ssd_validate_forward_ex(const ssd_dims *dims, const ssd_dt_options *opts,
                                   const void *x, const void *dt, const float *A, const void *B,
                                   const void *C, const float *D, const float *init_state,
                                   const void *y, const float *final_state, const void *workspace,
                                   size_t workspace_bytes);
ssd_status ssd_validate_backward(const ssd_dims *dims, const void *x, const void *dt,
                                 const float *A, const void *B, const void *C, const float *D,
                                 const float *init_state, const void *dy,
                                 const float *dfinal_state, const void *dx, const void *ddt,
                                 const float *dA, const void *dB, const void *dC, const float *dD,
                                 const float *dinit_state, const void *workspace,
                                 size_t workspace_bytes);

#ifdef __cplusplus
}
#endif
#endif /* SSD_MI355X_H */
