// C ABI of libssd_mi355x.so: argument validation, workspace layout and the
// launch sequence of each entry point.  The contract is documented in
// include/ssd.h.  Validation is pure host code (no HIP call), so it can be
// exercised on a machine without a GPU.
#include "ssd.h"

#include <hip/hip_runtime.h>

#include <cstdint>
#include <algorithm>
#include <cstring>

#include "ssd_internal.h"
#include "ssd_launch.h"

namespace {

constexpr int64_t kMaxGridYZ = 65535;
thread_local hipError_t g_last_hip = hipSuccess;

struct Range {
    uintptr_t lo = 0, hi = 0;  // [lo, hi); empty when lo == hi
    bool empty() const { return lo == hi; }
};

Range range_of(const void *p, int64_t bytes) {
    Range r;
    if (p && bytes > 0) {
        r.lo = (uintptr_t)p;
        r.hi = r.lo + (uintptr_t)bytes;
    }
    return r;
}

bool overlap(const Range &a, const Range &b) {
    return !a.empty() && !b.empty() && a.lo < b.hi && b.lo < a.hi;
}

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

// The integer a C caller stored in an enum-typed field or argument.  A C
// caller may pass any int there; reading it through the enum type is
// undefined in C++ when the value lies outside the enumeration, so its bytes
// are read as an int instead.
template <typename E> int raw_enum(const E &e) {
    static_assert(sizeof(E) == sizeof(int), "enums of the C ABI are int-sized");
    int v;
    std::memcpy(&v, &e, sizeof v);
    return v;
}

bool is_pow2_in(int64_t v, int64_t lo, int64_t hi) {
    return v >= lo && v <= hi && (v & (v - 1)) == 0;
}

// Multiplies with overflow detection; returns false past 2^62.
bool mul_ok(int64_t &acc, int64_t v) {
    if (v < 0) return false;
    if (v != 0 && acc > ((int64_t)1 << 62) / v) return false;
    acc *= v;
    return true;
}

ssd_status check_dims(const ssd_dims *d, bool decode, ssd::Dims *out) {
    if (!d) return SSD_ERR_NULL;
    if (raw_enum(d->dtype) != SSD_F32 && raw_enum(d->dtype) != SSD_BF16) return SSD_ERR_DTYPE;
    const int64_t L = decode ? 1 : d->seqlen;
    if (d->batch < 0 || L < 0 || d->nheads < 1 || d->headdim < 1 || d->dstate < 1 ||
        d->ngroups < 1 || (!decode && d->chunk < 1))
        return SSD_ERR_SHAPE;
    if (d->nheads % d->ngroups != 0) return SSD_ERR_SHAPE;
    if (!is_pow2_in(d->headdim, 16, 128) || !is_pow2_in(d->dstate, 16, 256))
        return SSD_ERR_UNSUPPORTED;
    if (!decode && (d->chunk % 16 != 0 || d->chunk > 256)) return SSD_ERR_UNSUPPORTED;
    if (d->batch > kMaxGridYZ || d->nheads > kMaxGridYZ) return SSD_ERR_UNSUPPORTED;
    const int64_t Q = decode ? 16 : d->chunk;
    const int64_t nc = (L + Q - 1) / Q;
    int64_t n = d->batch;  // largest array: x / y, or the chunk states
    if (!mul_ok(n, L) || !mul_ok(n, d->nheads) || !mul_ok(n, d->headdim))
        return SSD_ERR_UNSUPPORTED;
    int64_t ns = d->batch;
    if (!mul_ok(ns, nc) || !mul_ok(ns, d->nheads) || !mul_ok(ns, d->headdim) ||
        !mul_ok(ns, d->dstate))
        return SSD_ERR_UNSUPPORTED;
    int64_t grid = d->batch;  // one workgroup per (b, c, h)
    if (!mul_ok(grid, nc) || !mul_ok(grid, d->nheads) || grid > INT32_MAX)
        return SSD_ERR_UNSUPPORTED;
    if (out) {
        out->b = d->batch;
        out->L = L;
        out->H = d->nheads;
        out->P = d->headdim;
        out->N = d->dstate;
        out->G = d->ngroups;
        out->Q = Q;
        out->nc = nc;
        out->dtype = d->dtype;
    }
    return SSD_OK;
}

int64_t esize(const ssd::Dims &d) { return d.dtype == SSD_BF16 ? 2 : 4; }

int64_t align256(int64_t v) { return (v + 255) & ~(int64_t)255; }

// Workspace of the staged arrangement: cs | C B^T | chunk states | input
// scale of every step (used with Euler or zero-order-hold scaling).
struct WsLayout {
    int64_t cs = 0, cb = 0, S = 0, sc = 0, total = 0;
};

WsLayout ws_layout(const ssd::Dims &d) {
    WsLayout w;
    const int64_t cs_bytes = d.b * d.H * d.nc * d.Q * 4;
    const int64_t cb_bytes = d.b * d.nc * d.G * d.Q * d.Q * esize(d);
    const int64_t s_bytes = d.b * d.nc * d.H * d.P * d.N * 4;
    w.cs = 0;
    w.cb = align256(w.cs + cs_bytes);
    w.S = align256(w.cb + cb_bytes);
    w.sc = align256(w.S + s_bytes);
    w.total = align256(w.sc + cs_bytes);
    if (d.b == 0 || d.nc == 0) w.total = 0;
    return w;
}

// Workspace of the single-pass arrangement: fragment-ordered operands of
// every 32-step chunk and group | decay record of every chunk and head.
struct WalkLayout {
    int64_t ops = 0, rec = 0, total = 0;
};

WalkLayout walk_layout(const ssd::Dims &d) {
    WalkLayout w;
    const ssd::WalkBytes wb = ssd::walk_bytes(d);
    w.ops = 0;
    w.rec = align256(wb.ops);
    w.total = align256(w.rec + wb.rec);
    if (d.b == 0 || d.L == 0) w.total = 0;
    return w;
}

int64_t ws_total(const ssd::Dims &d) {
    int64_t t = ws_layout(d).total;
    if (ssd::walk_supported(d)) t = std::max(t, walk_layout(d).total);
    return t;
}

// Workspace of the gradient: cs | C B^T | (C B^T)^T | forward states H_c |
// state gradients R_c | dCB | dCB^T | state terms of dC and dB | per-chunk
// partials of dA and dD | float64 prefix (float32 inputs only) | C and B
// rows and the diagonal of C B^T in fragment order (when the chunk backward
// reads fragments; C B^T and its transpose are then fragment blocks too).
struct BwdLayout {
    int64_t cs = 0, cb = 0, cbT = 0, Hs = 0, Rs = 0, dcb = 0, dcbT = 0, dCs = 0, dBs = 0,
            part = 0, cs64 = 0, Cf = 0, Bf = 0, dg = 0, total = 0;
};

BwdLayout bwd_layout(const ssd::Dims &d) {
    BwdLayout w;
    const bool fr = ssd::chunk_bwd_frags(d);
    const ssd::BwdFragBytes fb = fr ? ssd::bwd_frag_bytes(d) : ssd::BwdFragBytes{0, 0, 0};
    const int64_t cb_bytes = fr ? fb.blocks : d.b * d.nc * d.G * d.Q * d.Q * esize(d);
    const int64_t s_bytes = d.b * d.nc * d.H * d.P * d.N * 4;
    const int64_t dcb_bytes = d.b * d.nc * d.G * d.Q * d.Q * 4;
    const int64_t g_bytes = d.b * d.L * d.G * d.N * 4;
    w.cs = 0;
    w.cb = align256(w.cs + d.b * d.H * d.nc * d.Q * 4);
    w.cbT = align256(w.cb + cb_bytes);
    w.Hs = align256(w.cbT + cb_bytes);
    w.Rs = align256(w.Hs + s_bytes);
    w.dcb = align256(w.Rs + s_bytes);
    w.dcbT = align256(w.dcb + dcb_bytes);
    w.dCs = align256(w.dcbT + dcb_bytes);
    w.dBs = align256(w.dCs + g_bytes);
    w.part = align256(w.dBs + g_bytes);
    w.cs64 = align256(w.part + d.b * d.nc * d.H * 2 * 4);
    w.Cf = align256(w.cs64 + (d.dtype == SSD_F32 ? d.b * d.H * d.nc * d.Q * 8 : 0));
    w.Bf = align256(w.Cf + fb.rows);
    w.dg = align256(w.Bf + fb.rows);
    w.total = align256(w.dg + fb.diag);
    if (d.b == 0 || d.nc == 0) w.total = 0;
    return w;
}

// Step-size options: validated, and converted for the kernels.  Inactive
// options (NULL, or all fields at their defaults) take the plain kernels.
bool opts_active(const ssd_dt_options *o) {
    return o && (o->dt_bias || o->dt_softplus || o->dt_max > o->dt_min || o->input_scale != SSD_SCALE_NONE);
}

ssd_status check_opts(const ssd_dt_options *o, const ssd::Dims &d) {
    if (!o) return SSD_OK;
    if (o->input_scale != SSD_SCALE_NONE && o->input_scale != SSD_SCALE_EULER &&
        o->input_scale != SSD_SCALE_ZOH)
        return SSD_ERR_UNSUPPORTED;
    if (o->dt_bias && ((uintptr_t)o->dt_bias % 16) != 0) return SSD_ERR_ALIGN;
    (void)d;
    return SSD_OK;
}

ssd::DtOpts to_dev(const ssd_dt_options *o) {
    return ssd::DtOpts{o->dt_bias, o->dt_min, o->dt_max, o->dt_softplus ? 1 : 0, (int)o->input_scale};
}

ssd_status hip_status(hipError_t e) {
    if (e == hipSuccess) return SSD_OK;
    g_last_hip = e;
    return SSD_ERR_HIP;
}

ssd_status validate_forward(const ssd_dims *dims, const void *x, const void *dt, const float *A,
                            const void *B, const void *C, const float *D, const float *init,
                            const void *y, const float *fin, const void *ws, size_t ws_bytes,
                            ssd::Dims *out) {
    ssd::Dims d;
    ssd_status st = check_dims(dims, false, &d);
    if (st != SSD_OK) return st;
    const bool tokens = d.b * d.L > 0;
    if (!A) return SSD_ERR_NULL;
    if (tokens && (!x || !dt || !B || !C || !y)) return SSD_ERR_NULL;
    const void *ptrs[] = {x, dt, A, B, C, D, init, y, fin};
    for (const void *p : ptrs)
        if (p && !aligned(p, 16)) return SSD_ERR_ALIGN;
    if (ws && !aligned(ws, 256)) return SSD_ERR_ALIGN;
    const int64_t wtotal = ws_total(d);
    if (wtotal > 0 && (!ws || (int64_t)ws_bytes < wtotal)) return SSD_ERR_WORKSPACE;
    const int64_t es = esize(d);
    const int64_t state_bytes = d.b * d.H * d.P * d.N * 4;
    const Range rx = range_of(x, d.b * d.L * d.H * d.P * es), rdt = range_of(dt, d.b * d.L * d.H * es),
                rA = range_of(A, d.H * 4), rB = range_of(B, d.b * d.L * d.G * d.N * es),
                rC = range_of(C, d.b * d.L * d.G * d.N * es), rD = range_of(D, d.H * 4),
                ri = range_of(init, state_bytes), ry = range_of(y, d.b * d.L * d.H * d.P * es),
                rf = range_of(fin, state_bytes), rw = range_of(ws, wtotal);
    const Range ins[] = {rx, rdt, rA, rB, rC, rD, ri};
    for (const Range &r : ins)
        if (overlap(ry, r) || overlap(rw, r)) return SSD_ERR_ALIAS;
    if (overlap(ry, rf) || overlap(ry, rw) || overlap(rf, rw)) return SSD_ERR_ALIAS;
    const Range ins_no_init[] = {rx, rdt, rA, rB, rC, rD};
    for (const Range &r : ins_no_init)
        if (overlap(rf, r)) return SSD_ERR_ALIAS;
    if (overlap(rf, ri) && (const void *)fin != (const void *)init) return SSD_ERR_ALIAS;
    if (out) *out = d;
    return SSD_OK;
}

ssd_status validate_decode(const ssd_dims *dims, const float *state, const void *x,
                           const void *dt, const float *A, const void *B, const void *C,
                           const float *D, const void *y, ssd::Dims *out) {
    ssd::Dims d;
    ssd_status st = check_dims(dims, true, &d);
    if (st != SSD_OK) return st;
    if (d.b * d.H * d.P > ssd::kDecodeMaxRows) return SSD_ERR_UNSUPPORTED;
    if (!A) return SSD_ERR_NULL;
    if (d.b > 0 && (!state || !x || !dt || !B || !C || !y)) return SSD_ERR_NULL;
    const void *ptrs[] = {state, x, dt, A, B, C, D, y};
    for (const void *p : ptrs)
        if (p && !aligned(p, 16)) return SSD_ERR_ALIGN;
    const int64_t es = esize(d);
    const Range rs = range_of(state, d.b * d.H * d.P * d.N * 4), rx = range_of(x, d.b * d.H * d.P * es),
                rdt = range_of(dt, d.b * d.H * es), rA = range_of(A, d.H * 4),
                rB = range_of(B, d.b * d.G * d.N * es), rC = range_of(C, d.b * d.G * d.N * es),
                rD = range_of(D, d.H * 4), ry = range_of(y, d.b * d.H * d.P * es);
    const Range ins[] = {rx, rdt, rA, rB, rC, rD};
    for (const Range &r : ins)
        if (overlap(ry, r) || overlap(rs, r)) return SSD_ERR_ALIAS;
    if (overlap(ry, rs)) return SSD_ERR_ALIAS;
    if (out) *out = d;
    return SSD_OK;
}

ssd_status validate_backward(const ssd_dims *dims, const void *x, const void *dt, const float *A,
                             const void *B, const void *C, const float *D, const float *init,
                             const void *dy, const float *dfinal, const void *dx, const void *ddt,
                             const float *dA, const void *dB, const void *dC, const float *dD,
                             const float *dinit, const void *ws, size_t ws_bytes, ssd::Dims *out) {
    ssd::Dims d;
    ssd_status st = check_dims(dims, false, &d);
    if (st != SSD_OK) return st;
    const bool tokens = d.b * d.L > 0;
    if (!A || !dA) return SSD_ERR_NULL;
    if (tokens && (!x || !dt || !B || !C || !dy || !dx || !ddt || !dB || !dC)) return SSD_ERR_NULL;
    const void *ptrs[] = {x, dt, A, B, C, D, init, dy, dfinal, dx, ddt, dA, dB, dC, dD, dinit};
    for (const void *p : ptrs)
        if (p && !aligned(p, 16)) return SSD_ERR_ALIGN;
    if (ws && !aligned(ws, 256)) return SSD_ERR_ALIGN;
    const int64_t wtotal = bwd_layout(d).total;
    if (wtotal > 0 && (!ws || (int64_t)ws_bytes < wtotal)) return SSD_ERR_WORKSPACE;
    const int64_t es = esize(d);
    const int64_t tok = d.b * d.L, state_bytes = d.b * d.H * d.P * d.N * 4;
    const Range ins[] = {range_of(x, tok * d.H * d.P * es), range_of(dt, tok * d.H * es),
                         range_of(A, d.H * 4),           range_of(B, tok * d.G * d.N * es),
                         range_of(C, tok * d.G * d.N * es), range_of(D, d.H * 4),
                         range_of(init, state_bytes),    range_of(dy, tok * d.H * d.P * es),
                         range_of(dfinal, state_bytes)};
    const Range outs[] = {range_of(dx, tok * d.H * d.P * es), range_of(ddt, tok * d.H * es),
                          range_of(dA, d.H * 4),           range_of(dB, tok * d.G * d.N * es),
                          range_of(dC, tok * d.G * d.N * es), range_of(dD, d.H * 4),
                          range_of(dinit, state_bytes),    range_of(ws, wtotal)};
    constexpr int nout = sizeof(outs) / sizeof(outs[0]);
    for (int i = 0; i < nout; ++i) {
        for (const Range &r : ins)
            if (overlap(outs[i], r)) return SSD_ERR_ALIAS;
        for (int j = i + 1; j < nout; ++j)
            if (overlap(outs[i], outs[j])) return SSD_ERR_ALIAS;
    }
    if (out) *out = d;
    return SSD_OK;
}

// Selective scan: shape checks, segment length and workspace.
ssd_status check_scan(const ssd_scan_dims *sd, ssd::ScanDims *out) {
    if (!sd) return SSD_ERR_NULL;
    if (raw_enum(sd->dtype) != SSD_F32 && raw_enum(sd->dtype) != SSD_BF16) return SSD_ERR_DTYPE;
    if (sd->batch < 0 || sd->seqlen < 0 || sd->channels < 1 || sd->ngroups < 1) return SSD_ERR_SHAPE;
    if (sd->channels % sd->ngroups != 0) return SSD_ERR_SHAPE;
    const int64_t N = sd->dstate;
    if (N != 4 && N != 8 && N != 16 && N != 32 && N != 64) return SSD_ERR_UNSUPPORTED;
    if (sd->ngroups > 1 && (sd->channels / sd->ngroups) % 64 != 0) return SSD_ERR_UNSUPPORTED;
    if (sd->batch > kMaxGridYZ || sd->channels > INT32_MAX / 64) return SSD_ERR_UNSUPPORTED;
    int64_t n = sd->batch;
    if (!mul_ok(n, sd->seqlen) || !mul_ok(n, sd->channels) || !mul_ok(n, N)) return SSD_ERR_UNSUPPORTED;
    if (sd->algo < 0 || sd->algo > 2) return SSD_ERR_UNSUPPORTED;
    // auto is segments: measured on the Mamba-2.8B layer shape (batch 4,
    // L 4096, 5120 channels, N 16, bf16) it takes 635 us against 684 us for
    // rows, whose per-lane B/C reads (two words per state update) load the
    // L1-to-register path as much as the arithmetic loads the ALUs
    const int64_t nblk = (sd->channels + 15) / 16;
    int algo = sd->algo == 0 ? 1 : sd->algo;
    if (algo == 2 && N != 16) return SSD_ERR_UNSUPPORTED;
    // rows: offsets within a batch row are 32-bit
    const bool rows_fit = sd->batch * nblk <= INT32_MAX && (sd->seqlen + 16) * sd->channels <= INT32_MAX;
    if (algo == 2 && !rows_fit) return SSD_ERR_UNSUPPORTED;
    const int64_t Lp = (sd->seqlen + 15) / 16 * 16;
    // segments: as many as fit one round of 8 waves per SIMD (8192 waves of
    // b x segments x 64-channel blocks), at least 32 steps each; pass 1 +
    // pass 3 cost the same for any segment length, and a second partial
    // round of waves would leave most SIMDs idle
    const int64_t cblk = (sd->channels + 63) / 64;
    const int64_t per_seg = std::max<int64_t>(sd->batch * cblk, 1);
    int64_t nseg = std::max<int64_t>(8192 / per_seg, 1);
    nseg = std::min<int64_t>(nseg, std::max<int64_t>((sd->seqlen + 31) / 32, 1));
    const int64_t seg = std::max<int64_t>((sd->seqlen + nseg - 1) / nseg, 1);
    nseg = (sd->seqlen + seg - 1) / seg;
    if (algo == 1 && nseg > kMaxGridYZ) return SSD_ERR_UNSUPPORTED;
    if (out)
        *out = ssd::ScanDims{sd->batch, sd->seqlen, sd->channels, N, sd->ngroups, seg, nseg, Lp, sd->dtype,
                             algo};
    return SSD_OK;
}

int64_t scan_ws_S(const ssd::ScanDims &d) {
    return d.algo == 2 ? 2 * d.b * d.G * d.N * d.Lp * 4 : d.b * d.nseg * d.Dch * d.N * 4;
}
int64_t scan_ws_total(const ssd::ScanDims &d) {
    if (d.b == 0 || d.L == 0) return 0;
    if (d.algo == 2) return align256(scan_ws_S(d));
    return align256(align256(scan_ws_S(d)) + d.b * d.nseg * d.Dch * 4);
}

ssd_status validate_scan(const ssd_scan_dims *sd, const void *x, const void *delta, const float *A,
                         const void *B, const void *C, const float *D, const void *z,
                         const float *dbias, const float *init, const void *y, const float *fin,
                         const void *ws, size_t ws_bytes, ssd::ScanDims *out) {
    ssd::ScanDims d;
    ssd_status st = check_scan(sd, &d);
    if (st != SSD_OK) return st;
    const bool tokens = d.b * d.L > 0;
    if (!A) return SSD_ERR_NULL;
    if (tokens && (!x || !delta || !B || !C || !y)) return SSD_ERR_NULL;
    const void *ptrs[] = {x, delta, A, B, C, D, z, dbias, init, y, fin};
    for (const void *p : ptrs)
        if (p && !aligned(p, 16)) return SSD_ERR_ALIGN;
    if (ws && !aligned(ws, 256)) return SSD_ERR_ALIGN;
    const int64_t wt = scan_ws_total(d);
    if (wt > 0 && (!ws || (int64_t)ws_bytes < wt)) return SSD_ERR_WORKSPACE;
    const int64_t es = d.dtype == SSD_BF16 ? 2 : 4;
    const int64_t tok = d.b * d.L * d.Dch * es, st_b = d.b * d.Dch * d.N * 4;
    const Range ins[] = {range_of(x, tok), range_of(delta, tok), range_of(A, d.Dch * d.N * 4),
                         range_of(B, d.b * d.L * d.G * d.N * es), range_of(C, d.b * d.L * d.G * d.N * es),
                         range_of(D, d.Dch * 4), range_of(z, tok), range_of(dbias, d.Dch * 4)};
    const Range ry = range_of(y, tok), rf = range_of(fin, st_b), ri = range_of(init, st_b),
                rw = range_of(ws, wt);
    for (const Range &r : ins)
        if (overlap(ry, r) || overlap(rf, r) || overlap(rw, r)) return SSD_ERR_ALIAS;
    if (overlap(ry, rf) || overlap(ry, rw) || overlap(rf, rw) || overlap(ry, ri) || overlap(rw, ri))
        return SSD_ERR_ALIAS;
    if (overlap(rf, ri) && (const void *)fin != (const void *)init) return SSD_ERR_ALIAS;
    if (out) *out = d;
    return SSD_OK;
}

ssd_status validate_ptrs(const void *const *req, int nreq, const void *const *opt, int nopt) {
    for (int i = 0; i < nreq; ++i)
        if (!req[i]) return SSD_ERR_NULL;
    for (int i = 0; i < nreq; ++i)
        if (!aligned(req[i], 16)) return SSD_ERR_ALIGN;
    for (int i = 0; i < nopt; ++i)
        if (opt[i] && !aligned(opt[i], 16)) return SSD_ERR_ALIGN;
    return SSD_OK;
}

// The five steps one after another, intermediates in the workspace.  With
// step-size options the prefix kernel preprocesses dt and (for Euler or
// zero-order-hold scaling) writes each step's input factor, which the
// chunk-state and scan kernels fold into their weights.
ssd_status run_staged(const ssd::Dims &d, const void *x, const void *dt, const float *A,
                      const void *B, const void *C, const float *D, const float *init, void *y,
                      float *fin, void *ws, hipStream_t st, const ssd::DtOpts *o = nullptr) {
    if (d.b == 0) return SSD_OK;
    if (d.nc == 0) return hip_status(ssd::launch_zero_state(d, init, fin, st));
    const WsLayout w = ws_layout(d);
    char *base = (char *)ws;
    float *cs = (float *)(base + w.cs);
    void *cb = base + w.cb;
    float *S = (float *)(base + w.S);
    float *sc = (o && o->scale != 0) ? (float *)(base + w.sc) : nullptr;
    hipError_t e;
    if (o) e = ssd::launch_chunk_cumsum_opts(d, dt, A, *o, cs, sc, st);
    else e = ssd::launch_chunk_cumsum(d, dt, A, cs, st);
    if (e != hipSuccess) return hip_status(e);
    if ((e = ssd::launch_chunk_cb(d, B, C, cb, nullptr, st)) != hipSuccess) return hip_status(e);
    if ((e = ssd::launch_chunk_state(d, x, B, cs, S, false, st, sc)) != hipSuccess) return hip_status(e);
    if ((e = ssd::launch_state_passing(d, S, cs, init, fin, st)) != hipSuccess) return hip_status(e);
    if ((e = ssd::launch_chunk_scan(d, x, C, cb, cs, S, D, y, st, sc)) != hipSuccess) return hip_status(e);
    return SSD_OK;
}

// Names of the kernel launches the gradient makes, in order.
const char *const kBwdNames[] = {"chunk_cumsum",      "chunk_cumsum64", "chunk_cb",
                                 "chunk_state",       "state_passing",  "chunk_state_rev",
                                 "state_passing_rev", "chunk_bwd",      "group_bwd",
                                 "group_combine",     "head_reduce"};
const char *const kBwdEmptyNames[] = {"copy_state", "head_reduce"};

int bwd_launches(const ssd::Dims &d, const char *const **names) {
    if (d.b == 0 || d.nc == 0) {
        if (names) *names = kBwdEmptyNames;
        return 2;
    }
    if (names) *names = kBwdNames;
    return 11;  // for bfloat16 inputs the chunk_cumsum64 slot launches nothing
}

// Records caller-supplied events around the launches (no-op without events).
struct Marks {
    void *const *ev;
    int n, k;
    hipStream_t st;
    hipError_t mark() {
        if (!ev || k >= n) return hipSuccess;
        return hipEventRecord((hipEvent_t)ev[k++], st);
    }
};

// The gradient: forward states recomputed, state gradients passed backwards,
// then the per-chunk and per-group gradient kernels.
ssd_status run_backward(const ssd::Dims &d, const void *x, const void *dt, const float *A,
                        const void *B, const void *C, const float *D, const float *init,
                        const void *dy, const float *dfinal, void *dx, void *ddt, float *dA,
                        void *dB, void *dC, float *dD, float *dinit, void *ws, hipStream_t st,
                        Marks mk) {
    hipError_t e;
#define SSD_STEP(call)                                                                            \
    do {                                                                                          \
        if ((e = (call)) != hipSuccess) return hip_status(e);                                     \
        if ((e = mk.mark()) != hipSuccess) return hip_status(e);                                  \
    } while (0)
    if ((e = mk.mark()) != hipSuccess) return hip_status(e);
    if (d.b == 0 || d.nc == 0) {
        SSD_STEP(ssd::launch_zero_state(d, dfinal, dinit, st));
        SSD_STEP(ssd::launch_head_reduce(d, nullptr, dA, dD, st));
        return SSD_OK;
    }
    const BwdLayout w = bwd_layout(d);
    char *base = (char *)ws;
    float *cs = (float *)(base + w.cs), *Hs = (float *)(base + w.Hs), *Rs = (float *)(base + w.Rs);
    float *dcb = (float *)(base + w.dcb), *dcbT = (float *)(base + w.dcbT);
    float *dCs = (float *)(base + w.dCs), *dBs = (float *)(base + w.dBs);
    float *part = (float *)(base + w.part);
    double *cs64 = d.dtype == SSD_F32 ? (double *)(base + w.cs64) : nullptr;
    void *cb = base + w.cb, *cbT = base + w.cbT;
    SSD_STEP(ssd::launch_chunk_cumsum(d, dt, A, cs, st));
    SSD_STEP(cs64 ? ssd::launch_chunk_cumsum64(d, dt, A, cs64, st) : hipSuccess);
    void *Cf = base + w.Cf, *Bf = base + w.Bf;
    float *dg = (float *)(base + w.dg);
    SSD_STEP(ssd::chunk_bwd_frags(d) ? ssd::launch_bwd_frags(d, B, C, cb, cbT, Cf, Bf, dg, st)
                                     : ssd::launch_chunk_cb(d, B, C, cb, cbT, st));
    SSD_STEP(ssd::launch_chunk_state(d, x, B, cs, Hs, false, st));
    SSD_STEP(ssd::launch_state_passing(d, Hs, cs, init, nullptr, st));
    SSD_STEP(ssd::launch_chunk_state(d, dy, C, cs, Rs, true, st));
    SSD_STEP(ssd::launch_state_passing_rev(d, Rs, cs, dfinal, dinit, st));
    SSD_STEP(ssd::launch_chunk_bwd(d, x, dy, dt, A, B, C, cb, cbT, Cf, Bf, dg, cs, cs64, Hs, Rs, D,
                                   dx, ddt, part, st));
    SSD_STEP(ssd::launch_group_bwd(d, x, dy, cs, cs64, Hs, Rs, dcb, dcbT, dCs, dBs, st));
    SSD_STEP(ssd::launch_group_combine(d, B, C, dcb, dcbT, dCs, dBs, dB, dC, st));
    SSD_STEP(ssd::launch_head_reduce(d, part, dA, dD, st));
#undef SSD_STEP
    return SSD_OK;
}

ssd_status run_walk_prep(const ssd::Dims &d, const void *dt, const float *A, const void *B, const void *C,
                         void *ws, hipStream_t st, const ssd::DtOpts *o = nullptr) {
    const WalkLayout w = walk_layout(d);
    char *base = (char *)ws;
    return hip_status(ssd::launch_walk_prep(d, dt, A, B, C, base + w.ops, (float *)(base + w.rec), st, o));
}

ssd_status run_walk_main(const ssd::Dims &d, const void *x, const float *D, const float *init, void *y,
                         float *fin, void *ws, hipStream_t st, bool opts = false) {
    const WalkLayout w = walk_layout(d);
    char *base = (char *)ws;
    return hip_status(ssd::launch_walk_main(d, x, base + w.ops, (const float *)(base + w.rec), D, init, y, fin,
                                            st, opts));
}

}  // namespace

namespace ssd {

ssd_status forward_dims_check(const ssd_dims *dims, size_t *ws_bytes) {
    ssd::Dims d;
    const ssd_status st = check_dims(dims, false, &d);
    if (st == SSD_OK && ws_bytes) *ws_bytes = (size_t)ws_total(d);
    return st;
}

ssd_status hip_error(hipError_t e) { return hip_status(e); }

}  // namespace ssd

extern "C" {

const char *ssd_status_string(ssd_status s) {
    switch (raw_enum(s)) {
    case SSD_OK: return "SSD_OK";
    case SSD_ERR_NULL: return "SSD_ERR_NULL: a required pointer is NULL";
    case SSD_ERR_SHAPE: return "SSD_ERR_SHAPE: negative or inconsistent sizes";
    case SSD_ERR_DTYPE: return "SSD_ERR_DTYPE: dtype must be SSD_F32 or SSD_BF16";
    case SSD_ERR_ALIGN: return "SSD_ERR_ALIGN: arrays must be 16-byte aligned (workspace 256-byte)";
    case SSD_ERR_WORKSPACE: return "SSD_ERR_WORKSPACE: workspace missing or too small";
    case SSD_ERR_UNSUPPORTED: return "SSD_ERR_UNSUPPORTED: shape outside the compiled set";
    case SSD_ERR_HIP: return "SSD_ERR_HIP: a HIP call or kernel launch failed";
    case SSD_ERR_ALIAS: return "SSD_ERR_ALIAS: an output overlaps an input";
    }
    return "SSD_ERR_UNKNOWN";
}

const char *ssd_last_hip_error(void) { return hipGetErrorString(g_last_hip); }

size_t ssd_forward_workspace_bytes(const ssd_dims *dims) {
    ssd::Dims d;
    if (check_dims(dims, false, &d) != SSD_OK) return 0;
    return (size_t)ws_total(d);
}

ssd_status ssd_validate_forward(const ssd_dims *dims, const void *x, const void *dt,
                                const float *A, const void *B, const void *C, const float *D,
                                const float *init_state, const void *y, const float *final_state,
                                const void *workspace, size_t workspace_bytes) {
    return validate_forward(dims, x, dt, A, B, C, D, init_state, y, final_state, workspace,
                            workspace_bytes, nullptr);
}

ssd_status ssd_validate_decode(const ssd_dims *dims, const float *state, const void *x,
                               const void *dt, const float *A, const void *B, const void *C,
                               const float *D, const void *y) {
    return validate_decode(dims, state, x, dt, A, B, C, D, y, nullptr);
}

// Validation shared by the forward entry points with options: the forward's
// checks, the options' own, and dt_bias kept clear of every output.
static ssd_status validate_forward_ex(const ssd_dims *dims, const ssd_dt_options *opts, const void *x,
                               const void *dt, const float *A, const void *B, const void *C,
                               const float *D, const float *init, const void *y, const float *fin,
                               const void *ws, size_t ws_bytes, ssd::Dims *out) {
    ssd::Dims d;
    ssd_status st = validate_forward(dims, x, dt, A, B, C, D, init, y, fin, ws, ws_bytes, &d);
    if (st != SSD_OK) return st;
    if ((st = check_opts(opts, d)) != SSD_OK) return st;
    if (opts && opts->dt_bias) {
        const Range rb = range_of(opts->dt_bias, d.H * 4);
        const int64_t es = esize(d);
        if (overlap(rb, range_of(y, d.b * d.L * d.H * d.P * es)) ||
            overlap(rb, range_of(fin, d.b * d.H * d.P * d.N * 4)) ||
            overlap(rb, range_of(ws, ws_total(d))))
            return SSD_ERR_ALIAS;
    }
    if (out) *out = d;
    return SSD_OK;
}

static ssd_status forward_any(const ssd_dims *dims, const ssd_dt_options *opts, bool staged_only,
                       const void *x, const void *dt, const float *A, const void *B, const void *C,
                       const float *D, const float *init_state, void *y, float *final_state,
                       void *workspace, size_t workspace_bytes, void *stream) {
    ssd::Dims d;
    ssd_status st = validate_forward_ex(dims, opts, x, dt, A, B, C, D, init_state, y, final_state,
                                        workspace, workspace_bytes, &d);
    if (st != SSD_OK) return st;
    ssd::DtOpts dev{};
    const ssd::DtOpts *o = nullptr;
    if (opts_active(opts)) {
        dev = to_dev(opts);
        o = &dev;
    }
    hipStream_t s = (hipStream_t)stream;
    if (!staged_only && d.b > 0 && d.L > 0 && ssd::walk_supported(d)) {
        if ((st = run_walk_prep(d, dt, A, B, C, workspace, s, o)) != SSD_OK) return st;
        return run_walk_main(d, x, D, init_state, y, final_state, workspace, s, o != nullptr);
    }
    return run_staged(d, x, dt, A, B, C, D, init_state, y, final_state, workspace, s, o);
}

ssd_status ssd_forward_staged(const ssd_dims *dims, const void *x, const void *dt,
                              const float *A, const void *B, const void *C, const float *D,
                              const float *init_state, void *y, float *final_state,
                              void *workspace, size_t workspace_bytes, void *stream) {
    return forward_any(dims, nullptr, true, x, dt, A, B, C, D, init_state, y, final_state,
                       workspace, workspace_bytes, stream);
}

ssd_status ssd_forward(const ssd_dims *dims, const void *x, const void *dt, const float *A,
                       const void *B, const void *C, const float *D, const float *init_state,
                       void *y, float *final_state, void *workspace, size_t workspace_bytes,
                       void *stream) {
    return forward_any(dims, nullptr, false, x, dt, A, B, C, D, init_state, y, final_state,
                       workspace, workspace_bytes, stream);
}

ssd_status ssd_forward_ex(const ssd_dims *dims, const ssd_dt_options *opts, const void *x,
                          const void *dt, const float *A, const void *B, const void *C,
                          const float *D, const float *init_state, void *y, float *final_state,
                          void *workspace, size_t workspace_bytes, void *stream) {
    return forward_any(dims, opts, false, x, dt, A, B, C, D, init_state, y, final_state,
                       workspace, workspace_bytes, stream);
}

ssd_status ssd_forward_staged_ex(const ssd_dims *dims, const ssd_dt_options *opts, const void *x,
                                 const void *dt, const float *A, const void *B, const void *C,
                                 const float *D, const float *init_state, void *y,
                                 float *final_state, void *workspace, size_t workspace_bytes,
                                 void *stream) {
    return forward_any(dims, opts, true, x, dt, A, B, C, D, init_state, y, final_state, workspace,
                       workspace_bytes, stream);
}

ssd_status ssd_validate_forward_ex(const ssd_dims *dims, const ssd_dt_options *opts,
                                   const void *x, const void *dt, const float *A, const void *B,
                                   const void *C, const float *D, const float *init_state,
                                   const void *y, const float *final_state, const void *workspace,
                                   size_t workspace_bytes) {
    return validate_forward_ex(dims, opts, x, dt, A, B, C, D, init_state, y, final_state,
                               workspace, workspace_bytes, nullptr);
}

int ssd_forward_is_single_pass(const ssd_dims *dims) {
    ssd::Dims d;
    if (check_dims(dims, false, &d) != SSD_OK) return 0;
    return (d.b > 0 && d.L > 0 && ssd::walk_supported(d)) ? 1 : 0;
}

ssd_status ssd_forward_prep(const ssd_dims *dims, const void *dt, const float *A, const void *B, const void *C,
                            void *workspace, size_t workspace_bytes, void *stream) {
    ssd::Dims d;
    ssd_status st = check_dims(dims, false, &d);
    if (st != SSD_OK) return st;
    if (!ssd::walk_supported(d)) return SSD_ERR_UNSUPPORTED;
    const void *req[] = {dt, A, B, C, workspace};
    if ((st = validate_ptrs(req, 5, nullptr, 0)) != SSD_OK) return st;
    if (!aligned(workspace, 256)) return SSD_ERR_ALIGN;
    if ((int64_t)workspace_bytes < ws_total(d)) return SSD_ERR_WORKSPACE;
    return run_walk_prep(d, dt, A, B, C, workspace, (hipStream_t)stream);
}

ssd_status ssd_forward_main(const ssd_dims *dims, const void *x, const void *dt, const float *A,
                            const void *B, const void *C, const float *D, const float *init_state,
                            void *y, float *final_state, void *workspace, size_t workspace_bytes,
                            void *stream) {
    ssd::Dims d;
    ssd_status st = validate_forward(dims, x, dt, A, B, C, D, init_state, y, final_state,
                                     workspace, workspace_bytes, &d);
    if (st != SSD_OK) return st;
    if (!ssd::walk_supported(d)) return SSD_ERR_UNSUPPORTED;
    return run_walk_main(d, x, D, init_state, y, final_state, workspace, (hipStream_t)stream);
}

ssd_status ssd_gated_rmsnorm(const ssd_dims *dims, int64_t norm_groups, float eps, const void *y,
                             const void *z, const float *weight, void *out, void *stream) {
    ssd::Dims d;
    ssd_status st = check_dims(dims, false, &d);
    if (st != SSD_OK) return st;
    const int64_t D = d.H * d.P;
    if (norm_groups < 1 || D % norm_groups != 0 || (D / norm_groups) % 8 != 0) return SSD_ERR_SHAPE;
    if (!(eps >= 0.f)) return SSD_ERR_SHAPE;
    if (d.b * d.L == 0) return SSD_OK;
    if (d.b * d.L > INT32_MAX) return SSD_ERR_UNSUPPORTED;
    const void *req[] = {y, z, weight, out};
    if ((st = validate_ptrs(req, 4, nullptr, 0)) != SSD_OK) return st;
    const int64_t bytes = d.b * d.L * D * esize(d);
    const Range ro = range_of(out, bytes), ry = range_of(y, bytes), rz = range_of(z, bytes),
                rw = range_of(weight, D * 4);
    if (overlap(ro, rz) || overlap(ro, rw) || (overlap(ro, ry) && out != y)) return SSD_ERR_ALIAS;
    return hip_status(
        ssd::launch_gated_rmsnorm(d, norm_groups, eps, y, z, weight, out, (hipStream_t)stream));
}

int32_t ssd_selective_scan_algo(const ssd_scan_dims *dims) {
    ssd::ScanDims d;
    const ssd_status st = check_scan(dims, &d);
    return st != SSD_OK ? -(int32_t)st : d.algo;
}

size_t ssd_selective_scan_workspace_bytes(const ssd_scan_dims *dims) {
    ssd::ScanDims d;
    if (check_scan(dims, &d) != SSD_OK) return 0;
    return (size_t)scan_ws_total(d);
}

ssd_status ssd_validate_selective_scan(const ssd_scan_dims *dims, const void *x, const void *delta,
                                       const float *A, const void *B, const void *C,
                                       const float *D, const void *z, const float *delta_bias,
                                       const float *init_state, const void *y,
                                       const float *final_state, const void *workspace,
                                       size_t workspace_bytes) {
    return validate_scan(dims, x, delta, A, B, C, D, z, delta_bias, init_state, y, final_state,
                         workspace, workspace_bytes, nullptr);
}

static ssd_status run_scan(const ssd_scan_dims *dims, const void *x, const void *delta,
                           const float *A, const void *B, const void *C, const float *D,
                           const void *z, const float *delta_bias, int32_t delta_softplus,
                           const float *init_state, void *y, float *final_state, void *workspace,
                           size_t workspace_bytes, void *stream, void *const *events,
                           int32_t n_events) {
    ssd::ScanDims d;
    ssd_status st = validate_scan(dims, x, delta, A, B, C, D, z, delta_bias, init_state, y,
                                  final_state, workspace, workspace_bytes, &d);
    if (st != SSD_OK) return st;
    if (n_events < 0 || (n_events > 0 && !events)) return SSD_ERR_NULL;
    float *S = (float *)workspace;
    float *sdl = (workspace && d.algo == 1) ? (float *)((char *)workspace + align256(scan_ws_S(d))) : nullptr;
    return hip_status(ssd::launch_selective_scan(d, x, delta, A, B, C, D, z, delta_bias,
                                                 delta_softplus ? 1 : 0, init_state, y,
                                                 final_state, S, sdl, (hipStream_t)stream, events,
                                                 n_events));
}

ssd_status ssd_selective_scan(const ssd_scan_dims *dims, const void *x, const void *delta,
                              const float *A, const void *B, const void *C, const float *D,
                              const void *z, const float *delta_bias, int32_t delta_softplus,
                              const float *init_state, void *y, float *final_state,
                              void *workspace, size_t workspace_bytes, void *stream) {
    return run_scan(dims, x, delta, A, B, C, D, z, delta_bias, delta_softplus, init_state, y,
                    final_state, workspace, workspace_bytes, stream, nullptr, 0);
}

ssd_status ssd_selective_scan_timed(const ssd_scan_dims *dims, const void *x, const void *delta,
                                    const float *A, const void *B, const void *C, const float *D,
                                    const void *z, const float *delta_bias, int32_t delta_softplus,
                                    const float *init_state, void *y, float *final_state,
                                    void *workspace, size_t workspace_bytes, void *stream,
                                    void *const *events, int32_t n_events) {
    return run_scan(dims, x, delta, A, B, C, D, z, delta_bias, delta_softplus, init_state, y,
                    final_state, workspace, workspace_bytes, stream, events, n_events);
}

size_t ssd_backward_workspace_bytes(const ssd_dims *dims) {
    ssd::Dims d;
    if (check_dims(dims, false, &d) != SSD_OK) return 0;
    return (size_t)bwd_layout(d).total;
}

ssd_status ssd_validate_backward(const ssd_dims *dims, const void *x, const void *dt,
                                 const float *A, const void *B, const void *C, const float *D,
                                 const float *init_state, const void *dy,
                                 const float *dfinal_state, const void *dx, const void *ddt,
                                 const float *dA, const void *dB, const void *dC, const float *dD,
                                 const float *dinit_state, const void *workspace,
                                 size_t workspace_bytes) {
    return validate_backward(dims, x, dt, A, B, C, D, init_state, dy, dfinal_state, dx, ddt, dA,
                             dB, dC, dD, dinit_state, workspace, workspace_bytes, nullptr);
}

ssd_status ssd_backward(const ssd_dims *dims, const void *x, const void *dt, const float *A,
                        const void *B, const void *C, const float *D, const float *init_state,
                        const void *dy, const float *dfinal_state, void *dx, void *ddt, float *dA,
                        void *dB, void *dC, float *dD, float *dinit_state, void *workspace,
                        size_t workspace_bytes, void *stream) {
    ssd::Dims d;
    ssd_status st = validate_backward(dims, x, dt, A, B, C, D, init_state, dy, dfinal_state, dx,
                                      ddt, dA, dB, dC, dD, dinit_state, workspace, workspace_bytes,
                                      &d);
    if (st != SSD_OK) return st;
    return run_backward(d, x, dt, A, B, C, D, init_state, dy, dfinal_state, dx, ddt, dA, dB, dC,
                        dD, dinit_state, workspace, (hipStream_t)stream,
                        Marks{nullptr, 0, 0, (hipStream_t)stream});
}

int ssd_backward_launch_count(const ssd_dims *dims) {
    ssd::Dims d;
    if (check_dims(dims, false, &d) != SSD_OK) return 0;
    return bwd_launches(d, nullptr);
}

const char *ssd_backward_launch_name(const ssd_dims *dims, int i) {
    ssd::Dims d;
    if (check_dims(dims, false, &d) != SSD_OK) return nullptr;
    const char *const *names = nullptr;
    const int n = bwd_launches(d, &names);
    return (i >= 0 && i < n) ? names[i] : nullptr;
}

ssd_status ssd_backward_timed(const ssd_dims *dims, const void *x, const void *dt, const float *A,
                              const void *B, const void *C, const float *D,
                              const float *init_state, const void *dy, const float *dfinal_state,
                              void *dx, void *ddt, float *dA, void *dB, void *dC, float *dD,
                              float *dinit_state, void *workspace, size_t workspace_bytes,
                              void *stream, void *const *events, int nevents) {
    ssd::Dims d;
    ssd_status st = validate_backward(dims, x, dt, A, B, C, D, init_state, dy, dfinal_state, dx,
                                      ddt, dA, dB, dC, dD, dinit_state, workspace, workspace_bytes,
                                      &d);
    if (st != SSD_OK) return st;
    if (!events) return SSD_ERR_NULL;
    if (nevents != bwd_launches(d, nullptr) + 1) return SSD_ERR_SHAPE;
    for (int i = 0; i < nevents; ++i)
        if (!events[i]) return SSD_ERR_NULL;
    return run_backward(d, x, dt, A, B, C, D, init_state, dy, dfinal_state, dx, ddt, dA, dB, dC,
                        dD, dinit_state, workspace, (hipStream_t)stream,
                        Marks{events, nevents, 0, (hipStream_t)stream});
}

ssd_status ssd_decode_step(const ssd_dims *dims, float *state, const void *x, const void *dt,
                           const float *A, const void *B, const void *C, const float *D, void *y,
                           void *stream) {
    return ssd_decode_step_ex(dims, nullptr, state, x, dt, A, B, C, D, y, stream);
}

ssd_status ssd_decode_step_ex(const ssd_dims *dims, const ssd_dt_options *opts, float *state,
                              const void *x, const void *dt, const float *A, const void *B,
                              const void *C, const float *D, void *y, void *stream) {
    ssd::Dims d;
    ssd_status st = validate_decode(dims, state, x, dt, A, B, C, D, y, &d);
    if (st != SSD_OK) return st;
    if ((st = check_opts(opts, d)) != SSD_OK) return st;
    if (opts && opts->dt_bias) {
        const Range rb = range_of(opts->dt_bias, d.H * 4);
        if (overlap(rb, range_of(state, d.b * d.H * d.P * d.N * 4)) ||
            overlap(rb, range_of(y, d.b * d.H * d.P * esize(d))))
            return SSD_ERR_ALIAS;
    }
    ssd::DtOpts dev{};
    const ssd::DtOpts *o = nullptr;
    if (opts_active(opts)) {
        dev = to_dev(opts);
        o = &dev;
    }
    return hip_status(ssd::launch_decode(d, state, x, dt, A, B, C, D, y, (hipStream_t)stream, o));
}

ssd_status ssd_chunk_cumsum(const ssd_dims *dims, const void *dt, const float *A, float *cs,
                            void *stream) {
    ssd::Dims d;
    ssd_status st = check_dims(dims, false, &d);
    if (st != SSD_OK) return st;
    if (d.b * d.nc == 0) return SSD_OK;
    const void *req[] = {dt, A, cs};
    if ((st = validate_ptrs(req, 3, nullptr, 0)) != SSD_OK) return st;
    return hip_status(ssd::launch_chunk_cumsum(d, dt, A, cs, (hipStream_t)stream));
}

ssd_status ssd_chunk_cb(const ssd_dims *dims, const void *B, const void *C, void *cb,
                        void *stream) {
    ssd::Dims d;
    ssd_status st = check_dims(dims, false, &d);
    if (st != SSD_OK) return st;
    if (d.b * d.nc == 0) return SSD_OK;
    const void *req[] = {B, C, cb};
    if ((st = validate_ptrs(req, 3, nullptr, 0)) != SSD_OK) return st;
    return hip_status(ssd::launch_chunk_cb(d, B, C, cb, nullptr, (hipStream_t)stream));
}

ssd_status ssd_chunk_state(const ssd_dims *dims, const void *x, const void *B, const float *cs,
                           float *states, void *stream) {
    ssd::Dims d;
    ssd_status st = check_dims(dims, false, &d);
    if (st != SSD_OK) return st;
    if (d.b * d.nc == 0) return SSD_OK;
    const void *req[] = {x, B, cs, states};
    if ((st = validate_ptrs(req, 4, nullptr, 0)) != SSD_OK) return st;
    return hip_status(ssd::launch_chunk_state(d, x, B, cs, states, false, (hipStream_t)stream));
}

ssd_status ssd_state_passing(const ssd_dims *dims, float *states, const float *cs,
                             const float *init_state, float *final_state, void *stream) {
    ssd::Dims d;
    ssd_status st = check_dims(dims, false, &d);
    if (st != SSD_OK) return st;
    if (d.b == 0) return SSD_OK;
    if (d.nc > 0) {
        const void *req[] = {states, cs};
        const void *opt[] = {init_state, final_state};
        if ((st = validate_ptrs(req, 2, opt, 2)) != SSD_OK) return st;
    } else {
        const void *opt[] = {init_state, final_state};
        if ((st = validate_ptrs(nullptr, 0, opt, 2)) != SSD_OK) return st;
    }
    const int64_t sb = d.b * d.H * d.P * d.N * 4;
    if (final_state && init_state != final_state &&
        overlap(range_of(final_state, sb), range_of(init_state, sb)))
        return SSD_ERR_ALIAS;
    return hip_status(
        ssd::launch_state_passing(d, states, cs, init_state, final_state, (hipStream_t)stream));
}

ssd_status ssd_chunk_scan(const ssd_dims *dims, const void *x, const void *C, const void *cb,
                          const float *cs, const float *hprev, const float *D, void *y,
                          void *stream) {
    ssd::Dims d;
    ssd_status st = check_dims(dims, false, &d);
    if (st != SSD_OK) return st;
    if (d.b * d.nc == 0) return SSD_OK;
    const void *req[] = {x, C, cb, cs, y};
    const void *opt[] = {hprev, D};
    if ((st = validate_ptrs(req, 5, opt, 2)) != SSD_OK) return st;
    const int64_t ybytes = d.b * d.L * d.H * d.P * esize(d);
    if (overlap(range_of(y, ybytes), range_of(x, ybytes))) return SSD_ERR_ALIAS;
    return hip_status(
        ssd::launch_chunk_scan(d, x, C, cb, cs, hprev, D, y, (hipStream_t)stream));
}

}  // extern "C"
