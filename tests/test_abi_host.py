"""Host-side checks of the C ABI (no GPU needed).

The library must load, export every function include/ssd.h declares, and
reject bad arguments on the host -- before any HIP call -- with the status
the header documents.  The validators never dereference the pointers, so
fake, suitably aligned addresses stand in for device buffers here.
"""
import ctypes
import subprocess

import pytest

import selective_state_space_04_amd as ssd

LIB = ssd.lib


def dims(**kw):
    base = dict(batch=2, seqlen=100, nheads=4, headdim=64, dstate=128, ngroups=2, chunk=64,
                dtype=ssd.BF16)
    base.update(kw)
    return ssd.make_dims(**base)


class Bufs:
    """Disjoint fake device ranges, 4 KiB aligned, far apart."""

    def __init__(self):
        self.next = 1 << 40

    def take(self, nbytes=0):
        p = self.next
        self.next += ((nbytes + (1 << 30)) >> 20) << 20
        return p


def fwd_args(d, **over):
    b = Bufs()
    ws = ssd.workspace_bytes(d)
    args = dict(x=b.take(), dt=b.take(), A=b.take(), B=b.take(), C=b.take(), D=b.take(), init=b.take(),
                y=b.take(), fin=b.take(), ws=b.take(), ws_bytes=ws)
    args.update(over)
    return args


def vfwd(d, a):
    return LIB.ssd_validate_forward(ctypes.byref(d), a["x"], a["dt"], a["A"], a["B"], a["C"], a["D"],
                                    a["init"], a["y"], a["fin"], a["ws"], a["ws_bytes"])


def test_exports_every_declared_symbol():
    names = ssd.header_functions()
    assert len(names) >= 13
    for n in names:
        assert hasattr(LIB, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", ssd.LIB_PATH], capture_output=True, text=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    assert set(names) <= exported


def test_status_strings():
    for code, name in ssd.STATUS.items():
        assert LIB.ssd_status_string(code).decode().startswith(name)
    assert LIB.ssd_status_string(99).decode() == "SSD_ERR_UNKNOWN"


def test_valid_forward_passes():
    d = dims()
    assert vfwd(d, fwd_args(d)) == 0
    assert vfwd(d, fwd_args(d, D=None, init=None, fin=None)) == 0


def test_workspace_bytes():
    al = lambda v: (v + 255) // 256 * 256
    # staged layout: cs | C B^T | chunk states | per-step input scale (as cs)
    d = dims(batch=2, seqlen=100, nheads=4, headdim=32, dstate=128, ngroups=2, chunk=64)
    nc = 2
    cs = 2 * 4 * nc * 64 * 4
    cb = 2 * nc * 2 * 64 * 64 * 2
    S = 2 * nc * 4 * 32 * 128 * 4
    staged = al(al(al(al(cs) + cb) + S) + cs)
    assert LIB.ssd_forward_is_single_pass(ctypes.byref(d)) == 0
    assert ssd.workspace_bytes(d) == staged
    # single-pass layout (bf16, P=64, N=128): per 32-step chunk and group the
    # C, B^T and causal C B^T fragments (18 KiB) | per chunk and head the decay
    # record (68 floats, the form with input scales); the workspace covers
    # both arrangements
    d = dims(batch=2, seqlen=100, nheads=4, headdim=64, dstate=128, ngroups=2, chunk=64)
    assert LIB.ssd_forward_is_single_pass(ctypes.byref(d)) == 1
    S = 2 * nc * 4 * 64 * 128 * 4
    staged = al(al(al(al(cs) + cb) + S) + cs)
    nblk = (100 + 31) // 32
    ops = 2 * nblk * 2 * 18432
    rec = 2 * nblk * 4 * 68 * 4
    fused = al(al(ops) + rec)
    assert ssd.workspace_bytes(d) == max(staged, fused)
    assert LIB.ssd_forward_is_single_pass(ctypes.byref(dims(dtype=ssd.F32))) == 0
    assert ssd.workspace_bytes(dims(seqlen=0)) == 0
    assert ssd.workspace_bytes(dims(headdim=48)) == 0


@pytest.mark.parametrize("field,value,status", [
    ("dtype", 2, "SSD_ERR_DTYPE"),
    ("batch", -1, "SSD_ERR_SHAPE"),
    ("seqlen", -5, "SSD_ERR_SHAPE"),
    ("nheads", 0, "SSD_ERR_SHAPE"),
    ("ngroups", 3, "SSD_ERR_SHAPE"),
    ("chunk", 0, "SSD_ERR_SHAPE"),
    ("headdim", 48, "SSD_ERR_UNSUPPORTED"),
    ("headdim", 256, "SSD_ERR_UNSUPPORTED"),
    ("dstate", 8, "SSD_ERR_UNSUPPORTED"),
    ("dstate", 512, "SSD_ERR_UNSUPPORTED"),
    ("chunk", 24, "SSD_ERR_UNSUPPORTED"),
    ("chunk", 512, "SSD_ERR_UNSUPPORTED"),
    ("batch", 70000, "SSD_ERR_UNSUPPORTED"),
])
def test_bad_dims(field, value, status):
    d = dims(**{field: value})
    good = dims()
    a = fwd_args(good)
    assert ssd.STATUS[vfwd(d, a)] == status


def test_null_dims():
    a = fwd_args(dims())
    assert LIB.ssd_validate_forward(None, a["x"], a["dt"], a["A"], a["B"], a["C"], a["D"], a["init"],
                                    a["y"], a["fin"], a["ws"], a["ws_bytes"]) == 1


@pytest.mark.parametrize("name", ["x", "dt", "A", "B", "C", "y"])
def test_null_required(name):
    d = dims()
    assert ssd.STATUS[vfwd(d, fwd_args(d, **{name: None}))] == "SSD_ERR_NULL"


def test_empty_sequence_allows_null_arrays():
    d = dims(seqlen=0)
    assert vfwd(d, fwd_args(d, x=None, dt=None, B=None, C=None, y=None, ws=None, ws_bytes=0)) == 0


@pytest.mark.parametrize("name", ["x", "dt", "A", "B", "C", "D", "init", "y", "fin"])
def test_misaligned(name):
    d = dims()
    a = fwd_args(d)
    a[name] += 8
    assert ssd.STATUS[vfwd(d, a)] == "SSD_ERR_ALIGN"


def test_workspace_checks():
    d = dims()
    a = fwd_args(d)
    assert ssd.STATUS[vfwd(d, dict(a, ws_bytes=a["ws_bytes"] - 1))] == "SSD_ERR_WORKSPACE"
    assert ssd.STATUS[vfwd(d, dict(a, ws=None))] == "SSD_ERR_WORKSPACE"
    assert ssd.STATUS[vfwd(d, dict(a, ws=a["ws"] + 128))] == "SSD_ERR_ALIGN"


def test_aliasing():
    d = dims()
    a = fwd_args(d)
    assert ssd.STATUS[vfwd(d, dict(a, y=a["x"]))] == "SSD_ERR_ALIAS"
    assert ssd.STATUS[vfwd(d, dict(a, y=a["C"] + 16))] == "SSD_ERR_ALIAS"
    assert ssd.STATUS[vfwd(d, dict(a, fin=a["D"]))] == "SSD_ERR_ALIAS"
    assert ssd.STATUS[vfwd(d, dict(a, ws=a["x"]))] == "SSD_ERR_ALIAS"
    # final_state may be init_state itself, but not a shifted view of it
    assert vfwd(d, dict(a, fin=a["init"])) == 0
    assert ssd.STATUS[vfwd(d, dict(a, fin=a["init"] + 256))] == "SSD_ERR_ALIAS"


def test_decode_validation():
    d = dims(seqlen=1)
    b = Bufs()
    ptrs = [b.take() for _ in range(8)]   # state, x, dt, A, B, C, D, y
    v = lambda dd, p: LIB.ssd_validate_decode(ctypes.byref(dd), *p)
    assert v(d, ptrs) == 0
    assert v(d, ptrs[:6] + [None] + ptrs[7:]) == 0          # D nullable
    for i in [0, 1, 2, 3, 4, 5, 7]:
        p = list(ptrs)
        p[i] = None
        assert ssd.STATUS[v(d, p)] == "SSD_ERR_NULL", i
    p = list(ptrs)
    p[7] = p[0]                                             # y aliases state
    assert ssd.STATUS[v(d, p)] == "SSD_ERR_ALIAS"
    p = list(ptrs)
    p[1] += 2
    assert ssd.STATUS[v(d, p)] == "SSD_ERR_ALIGN"
    assert ssd.STATUS[v(dims(dstate=24), ptrs)] == "SSD_ERR_UNSUPPORTED"
    # the decode kernels index state rows with 32 bits: batch * H * P must stay
    # below 2^31 - 4096 (checked on the sizes alone, before any pointer)
    lim = (1 << 31) - 4096
    bmax, P = 65535, 64                     # batch at its own limit (the grid's)
    h_ok = lim // (bmax * P)
    assert bmax * h_ok * P <= lim < bmax * (h_ok + 1) * P
    assert ssd.STATUS[v(dims(batch=bmax, seqlen=1, nheads=h_ok + 1, headdim=P, ngroups=1), [None] * 8)] == \
        "SSD_ERR_UNSUPPORTED"
    assert ssd.STATUS[v(dims(batch=bmax, seqlen=1, nheads=h_ok, headdim=P, ngroups=1), [None] * 8)] == \
        "SSD_ERR_NULL"


def test_entry_points_reject_before_launch():
    """Errors come back from the real entry points without touching a device."""
    d = dims(headdim=48)
    a = fwd_args(dims())
    st = LIB.ssd_forward(ctypes.byref(d), a["x"], a["dt"], a["A"], a["B"], a["C"], a["D"], a["init"],
                         a["y"], a["fin"], a["ws"], a["ws_bytes"], None)
    assert ssd.STATUS[st] == "SSD_ERR_UNSUPPORTED"
    assert ssd.STATUS[LIB.ssd_chunk_cumsum(ctypes.byref(dims()), None, a["A"], a["ws"], None)] == "SSD_ERR_NULL"
    assert ssd.STATUS[LIB.ssd_chunk_scan(ctypes.byref(dims()), a["x"], a["C"], a["ws"], a["ws"], None, None,
                                         a["x"], None)] == "SSD_ERR_ALIAS"
    assert ssd.STATUS[LIB.ssd_decode_step(ctypes.byref(dims(dtype=5)), *([a["x"]] * 8), None, None)] == \
        "SSD_ERR_DTYPE"


def test_noalloc_rejects_before_any_hip_call():
    """The no-allocation forward rejects bad dims, and dims whose workspace
    exceeds its fixed array, on the host (this machine has no GPU: any HIP
    call would fail with SSD_ERR_HIP instead)."""
    a = fwd_args(dims())
    ptrs = [a[k] for k in ("x", "dt", "A", "B", "C", "D", "init", "y", "fin")]
    bad = dims(headdim=48)
    assert ssd.STATUS[LIB.ssd_forward_noalloc(ctypes.byref(bad), *ptrs, None)] == "SSD_ERR_UNSUPPORTED"
    big = dims(batch=1, seqlen=65536, nheads=32, ngroups=1, chunk=256, dtype=ssd.F32)
    assert ssd.workspace_bytes(big) > ssd.NOALLOC_WORKSPACE_BYTES
    assert ssd.STATUS[LIB.ssd_forward_noalloc(ctypes.byref(big), *ptrs, None)] == "SSD_ERR_WORKSPACE"
    assert ssd.STATUS[LIB.ssd_forward_noalloc(None, *ptrs, None)] == "SSD_ERR_NULL"


# ------------------------------------------------------------------ backward
BWD_NAMES = ["x", "dt", "A", "B", "C", "D", "init", "dy", "dfinal", "dx", "ddt", "dA", "dB", "dC", "dD",
             "dinit"]


def bwd_args(d, **over):
    b = Bufs()
    args = {k: b.take() for k in BWD_NAMES}
    args["ws"] = b.take()
    args["ws_bytes"] = ssd.backward_workspace_bytes(d)
    args.update(over)
    return args


def vbwd(d, a):
    return LIB.ssd_validate_backward(ctypes.byref(d), *[a[k] for k in BWD_NAMES], a["ws"], a["ws_bytes"])


def test_backward_valid_and_nullable():
    d = dims()
    assert vbwd(d, bwd_args(d)) == 0
    assert vbwd(d, bwd_args(d, D=None, init=None, dfinal=None, dD=None, dinit=None)) == 0


@pytest.mark.parametrize("name", ["x", "dt", "A", "B", "C", "dy", "dx", "ddt", "dA", "dB", "dC"])
def test_backward_null_required(name):
    d = dims()
    assert ssd.STATUS[vbwd(d, bwd_args(d, **{name: None}))] == "SSD_ERR_NULL"


@pytest.mark.parametrize("name", BWD_NAMES)
def test_backward_misaligned(name):
    d = dims()
    a = bwd_args(d)
    a[name] += 4
    assert ssd.STATUS[vbwd(d, a)] == "SSD_ERR_ALIGN"


def test_backward_workspace_and_alias():
    d = dims()
    a = bwd_args(d)
    assert ssd.STATUS[vbwd(d, dict(a, ws_bytes=a["ws_bytes"] - 1))] == "SSD_ERR_WORKSPACE"
    assert ssd.STATUS[vbwd(d, dict(a, ws=None))] == "SSD_ERR_WORKSPACE"
    assert ssd.STATUS[vbwd(d, dict(a, dx=a["x"]))] == "SSD_ERR_ALIAS"        # output over an input
    assert ssd.STATUS[vbwd(d, dict(a, dB=a["dC"] + 16))] == "SSD_ERR_ALIAS"  # two outputs overlap
    assert ssd.STATUS[vbwd(d, dict(a, dinit=a["dfinal"]))] == "SSD_ERR_ALIAS"
    assert ssd.STATUS[vbwd(d, dict(a, ws=a["dy"]))] == "SSD_ERR_ALIAS"
    assert ssd.STATUS[vbwd(dims(headdim=48), a)] == "SSD_ERR_UNSUPPORTED"


def test_backward_empty_allows_null_arrays():
    d = dims(seqlen=0)
    assert ssd.backward_workspace_bytes(d) == 0
    a = bwd_args(d, x=None, dt=None, B=None, C=None, dy=None, dx=None, ddt=None, dB=None, dC=None, ws=None,
                 ws_bytes=0)
    assert vbwd(d, a) == 0


def test_backward_workspace_bytes():
    b, L, H, P, N, G, Q = 2, 100, 4, 64, 128, 2, 64
    nc = 2
    al = lambda v: (v + 255) & ~255
    # bfloat16: C B^T and its transpose as fragment blocks (per (b, c, g): Q / 16 row tiles x 8
    # blocks of 1 KiB), then the C and B rows in fragment order (Q / 16 x ceil(N / 32) blocks of
    # 1 KiB each) and the float32 diagonal of C B^T
    nbcg, t16, ncf = b * nc * G, Q // 16, (N + 31) // 32
    o = 0
    for nbytes in [b * H * nc * Q * 4, nbcg * t16 * 8 * 1024, nbcg * t16 * 8 * 1024, b * nc * H * P * N * 4,
                   b * nc * H * P * N * 4, b * nc * G * Q * Q * 4, b * nc * G * Q * Q * 4, b * L * G * N * 4,
                   b * L * G * N * 4, b * nc * H * 2 * 4, 0, nbcg * t16 * ncf * 1024, nbcg * t16 * ncf * 1024,
                   nbcg * Q * 4]:
        o = al(o + nbytes)
    assert ssd.backward_workspace_bytes(dims()) == o
    # float32 inputs add a float64 decay prefix
    o32 = 0
    for nbytes in [b * H * nc * Q * 4, b * nc * G * Q * Q * 4, b * nc * G * Q * Q * 4, b * nc * H * P * N * 4,
                   b * nc * H * P * N * 4, b * nc * G * Q * Q * 4, b * nc * G * Q * Q * 4, b * L * G * N * 4,
                   b * L * G * N * 4, b * nc * H * 2 * 4, b * H * nc * Q * 8]:
        o32 = al(o32 + nbytes)
    assert ssd.backward_workspace_bytes(dims(dtype=ssd.F32)) == o32
    assert ssd.backward_workspace_bytes(dims(headdim=48)) == 0


# ------------------------------------------------------------------ step-size options
def vfwd_ex(d, opts, a):
    return LIB.ssd_validate_forward_ex(ctypes.byref(d), None if opts is None else ctypes.byref(opts), a["x"], a["dt"],
                                       a["A"], a["B"], a["C"], a["D"], a["init"], a["y"], a["fin"], a["ws"],
                                       a["ws_bytes"])


def test_forward_ex_options_validation():
    d = dims()
    a = fwd_args(d)
    bias = Bufs().take() + (1 << 45)
    assert vfwd_ex(d, None, a) == 0
    assert vfwd_ex(d, ssd.DtOptions(bias, 1, 0.0, 0.0, 2), a) == 0
    assert ssd.STATUS[vfwd_ex(d, ssd.DtOptions(None, 0, 0.0, 0.0, 3), a)] == "SSD_ERR_UNSUPPORTED"
    assert ssd.STATUS[vfwd_ex(d, ssd.DtOptions(bias + 4, 0, 0.0, 0.0, 0), a)] == "SSD_ERR_ALIGN"
    assert ssd.STATUS[vfwd_ex(d, ssd.DtOptions(a["y"], 1, 0.0, 0.0, 0), a)] == "SSD_ERR_ALIAS"
    assert ssd.STATUS[vfwd_ex(d, ssd.DtOptions(a["ws"] + 256, 1, 0.0, 0.0, 0), a)] == "SSD_ERR_ALIAS"
    # the forward's own checks still apply
    assert ssd.STATUS[vfwd_ex(d, ssd.DtOptions(bias, 1, 0.0, 0.0, 1), dict(a, x=None))] == "SSD_ERR_NULL"


def test_make_options_defaults_are_the_plain_map():
    import torch
    A = torch.zeros(4)
    assert ssd.make_options(A) is None
    o = ssd.make_options(A, dt_softplus=True, dt_limit=(0.001, 0.5), input_scale="zoh")
    assert (o.dt_softplus, o.input_scale) == (1, 2) and abs(o.dt_max - 0.5) < 1e-7
    with pytest.raises(ValueError):
        ssd.make_options(A, input_scale="bilinear")


def test_gated_rmsnorm_validation():
    d = dims()                                     # H * P = 256
    b = Bufs()
    y, z, w, out = b.take(), b.take(), b.take(), b.take()
    f = lambda dd, g, e, *p: ssd.STATUS[LIB.ssd_gated_rmsnorm(ctypes.byref(dd), g, e, *p, None)]
    assert f(d, 3, 1e-5, y, z, w, out) == "SSD_ERR_SHAPE"          # 3 does not divide 256
    assert f(d, 64, 1e-5, y, z, w, out) == "SSD_ERR_SHAPE"         # groups of 4 channels
    assert f(d, 1, -1.0, y, z, w, out) == "SSD_ERR_SHAPE"
    assert f(d, 1, 1e-5, y, z, None, out) == "SSD_ERR_NULL"
    assert f(d, 1, 1e-5, y, z, w, z) == "SSD_ERR_ALIAS"
    assert f(d, 1, 1e-5, y, z, w, y + 16) == "SSD_ERR_ALIAS"
    assert f(d, 1, 1e-5, y + 8, z, w, out) == "SSD_ERR_ALIGN"
    assert f(dims(seqlen=0), 1, 1e-5, None, None, None, None) == "SSD_OK"


def test_selective_scan_validation():
    sd = lambda **kw: ssd.ScanDims(**{**dict(batch=2, seqlen=300, channels=128, dstate=16, ngroups=1,
                                            dtype=ssd.BF16), **kw})
    b = Bufs()
    p = {k: b.take() for k in ("x", "dl", "A", "B", "C", "D", "z", "bias", "init", "y", "fin", "ws")}
    d = sd()
    wsb = LIB.ssd_selective_scan_workspace_bytes(ctypes.byref(d))
    assert wsb > 0
    v = lambda dd, **o: ssd.STATUS[LIB.ssd_validate_selective_scan(
        ctypes.byref(dd), *[o.get(k, p[k]) for k in ("x", "dl", "A", "B", "C", "D", "z", "bias", "init", "y", "fin",
                                                     "ws")], o.get("wsb", wsb))]
    assert v(d) == "SSD_OK"
    assert v(d, D=None, z=None, bias=None, init=None, fin=None) == "SSD_OK"
    assert v(sd(dstate=12)) == "SSD_ERR_UNSUPPORTED"
    assert v(sd(ngroups=2, channels=96)) == "SSD_ERR_UNSUPPORTED"      # 48 channels per group
    assert v(sd(ngroups=3)) == "SSD_ERR_SHAPE"
    assert v(sd(dtype=7)) == "SSD_ERR_DTYPE"
    assert v(d, x=None) == "SSD_ERR_NULL"
    assert v(d, y=p["x"]) == "SSD_ERR_ALIAS"
    assert v(d, fin=p["init"]) == "SSD_OK"                              # in-place carry
    assert v(d, fin=p["init"] + 64) == "SSD_ERR_ALIAS"
    assert v(d, wsb=wsb - 1) == "SSD_ERR_WORKSPACE"
    assert v(d, z=p["z"] + 2) == "SSD_ERR_ALIGN"
    assert LIB.ssd_selective_scan_workspace_bytes(ctypes.byref(sd(seqlen=0))) == 0
    # arrangements: rows needs N = 16; the workspace follows the choice
    assert v(sd(algo=2)) in ("SSD_OK", "SSD_ERR_WORKSPACE")
    assert v(sd(algo=2, dstate=8)) == "SSD_ERR_UNSUPPORTED"
    assert v(sd(algo=3)) == "SSD_ERR_UNSUPPORTED"
    rows = LIB.ssd_selective_scan_workspace_bytes(ctypes.byref(sd(algo=2)))
    assert rows == 2 * 2 * 1 * 16 * 304 * 4                      # B and C as float32 [b, G, N, 304]
    assert LIB.ssd_selective_scan_workspace_bytes(ctypes.byref(sd(algo=1))) == wsb
    assert LIB.ssd_selective_scan_algo(ctypes.byref(sd(batch=4, seqlen=4096, channels=5120))) == 1
    assert LIB.ssd_selective_scan_algo(ctypes.byref(sd(algo=2))) == 2
    assert LIB.ssd_selective_scan_algo(ctypes.byref(sd(algo=2, dstate=8))) < 0
    # segments: as many as fit 8192 waves, at least 32 steps each
    big = sd(batch=4, seqlen=4096, channels=5120, algo=1)            # 4 x 80 blocks -> 25 segments of 164
    al = lambda v: (v + 255) // 256 * 256
    states, sums = 4 * 25 * 5120 * 16 * 4, 4 * 25 * 5120 * 4     # segment end states, step sums
    assert LIB.ssd_selective_scan_workspace_bytes(ctypes.byref(big)) == al(al(states) + sums)
