"""MI355X (gfx950) SSD layer: Python binding of libssd_mi355x.so.

This module only marshals arguments: it checks tensor devices, dtypes,
shapes and contiguity, allocates outputs (and the workspace unless one is
passed), and calls the C ABI declared in ``include/ssd.h`` on the current
torch stream.  Every step of the computation runs in the library's HIP
kernels; there is no fallback.  Importing fails loudly when the library has
not been built (``python selective_state_space_04_amd/build.py``).

Layouts: x, y [b, L, H, P]; dt [b, L, H]; B, C [b, L, G, N]; A, D [H] float32;
states [b, H, P, N] float32.  x, dt, B, C share one dtype (float32 or
bfloat16), which is also y's dtype.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libssd_mi355x.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "ssd.h")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with "
                      "`python selective_state_space_04_amd/build.py` (hipcc, gfx950)")


class Dims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64), ("nheads", ctypes.c_int64),
                ("headdim", ctypes.c_int64), ("dstate", ctypes.c_int64), ("ngroups", ctypes.c_int64),
                ("chunk", ctypes.c_int64), ("dtype", ctypes.c_int32)]


class DtOptions(ctypes.Structure):
    """ssd_dt_options: step-size bias/softplus/clamp and the input scale."""
    _fields_ = [("dt_bias", ctypes.c_void_p), ("dt_softplus", ctypes.c_int32), ("dt_min", ctypes.c_float),
                ("dt_max", ctypes.c_float), ("input_scale", ctypes.c_int32)]


SCALES = {"none": 0, "euler": 1, "zoh": 2}
F32, BF16 = 0, 1
_DT = {torch.float32: F32, torch.bfloat16: BF16}
STATUS = {0: "SSD_OK", 1: "SSD_ERR_NULL", 2: "SSD_ERR_SHAPE", 3: "SSD_ERR_DTYPE", 4: "SSD_ERR_ALIGN",
          5: "SSD_ERR_WORKSPACE", 6: "SSD_ERR_UNSUPPORTED", 7: "SSD_ERR_HIP", 8: "SSD_ERR_ALIAS"}

_vp, _dp = ctypes.c_void_p, ctypes.POINTER(Dims)
lib = ctypes.CDLL(LIB_PATH)
_SIGS = {
    "ssd_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "ssd_last_hip_error": (ctypes.c_char_p, []),
    "ssd_forward_workspace_bytes": (ctypes.c_size_t, [_dp]),
    "ssd_forward": (ctypes.c_int, [_dp] + [_vp] * 10 + [ctypes.c_size_t, _vp]),
    "ssd_forward_staged": (ctypes.c_int, [_dp] + [_vp] * 10 + [ctypes.c_size_t, _vp]),
    "ssd_decode_step": (ctypes.c_int, [_dp] + [_vp] * 9),
    "ssd_forward_is_single_pass": (ctypes.c_int, [_dp]),
    "ssd_forward_prep": (ctypes.c_int, [_dp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]),
    "ssd_forward_main": (ctypes.c_int, [_dp] + [_vp] * 10 + [ctypes.c_size_t, _vp]),
    "ssd_forward_noalloc": (ctypes.c_int, [_dp] + [_vp] * 10),
    "ssd_chunk_cumsum": (ctypes.c_int, [_dp, _vp, _vp, _vp, _vp]),
    "ssd_chunk_cb": (ctypes.c_int, [_dp, _vp, _vp, _vp, _vp]),
    "ssd_chunk_state": (ctypes.c_int, [_dp, _vp, _vp, _vp, _vp, _vp]),
    "ssd_state_passing": (ctypes.c_int, [_dp, _vp, _vp, _vp, _vp, _vp]),
    "ssd_chunk_scan": (ctypes.c_int, [_dp] + [_vp] * 8),
    "ssd_validate_forward": (ctypes.c_int, [_dp] + [_vp] * 10 + [ctypes.c_size_t]),
    "ssd_validate_decode": (ctypes.c_int, [_dp] + [_vp] * 8),
    "ssd_backward_workspace_bytes": (ctypes.c_size_t, [_dp]),
    "ssd_backward": (ctypes.c_int, [_dp] + [_vp] * 17 + [ctypes.c_size_t, _vp]),
    "ssd_validate_backward": (ctypes.c_int, [_dp] + [_vp] * 17 + [ctypes.c_size_t]),
    "ssd_forward_ex": (ctypes.c_int, [_dp, _vp] + [_vp] * 10 + [ctypes.c_size_t, _vp]),
    "ssd_forward_staged_ex": (ctypes.c_int, [_dp, _vp] + [_vp] * 10 + [ctypes.c_size_t, _vp]),
    "ssd_decode_step_ex": (ctypes.c_int, [_dp, _vp] + [_vp] * 9),
    "ssd_validate_forward_ex": (ctypes.c_int, [_dp, _vp] + [_vp] * 10 + [ctypes.c_size_t]),
    "ssd_gated_rmsnorm": (ctypes.c_int, [_dp, ctypes.c_int64, ctypes.c_float] + [_vp] * 5),
    "ssd_selective_scan_workspace_bytes": (ctypes.c_size_t, [ctypes.c_void_p]),
    "ssd_selective_scan_algo": (ctypes.c_int32, [ctypes.c_void_p]),
    "ssd_selective_scan": (ctypes.c_int, [_vp] * 9 + [ctypes.c_int32] + [_vp] * 4 + [ctypes.c_size_t, _vp]),
    "ssd_validate_selective_scan": (ctypes.c_int, [_vp] * 13 + [ctypes.c_size_t]),
    "ssd_selective_scan_timed": (ctypes.c_int, [_vp] * 9 + [ctypes.c_int32] + [_vp] * 4
                                 + [ctypes.c_size_t, _vp, _vp, ctypes.c_int32]),
    "ssd_backward_launch_count": (ctypes.c_int, [_dp]),
    "ssd_backward_launch_name": (ctypes.c_char_p, [_dp, ctypes.c_int]),
    "ssd_backward_timed": (ctypes.c_int, [_dp] + [_vp] * 17 + [ctypes.c_size_t, _vp, _vp, ctypes.c_int]),
}
for _name, (_res, _args) in _SIGS.items():
    _f = getattr(lib, _name)
    _f.restype, _f.argtypes = _res, _args


def header_functions() -> list[str]:
    """Names of the functions include/ssd.h declares."""
    text = open(HEADER_PATH).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(ssd_\w+)\s*\(", text, re.M)))


class SSDError(RuntimeError):
    def __init__(self, status: int):
        msg = lib.ssd_status_string(status).decode()
        if status == 7:
            msg += f" ({lib.ssd_last_hip_error().decode()})"
        super().__init__(msg)
        self.status = status
        self.name = STATUS.get(status, str(status))


def _check(status: int) -> None:
    if status != 0:
        raise SSDError(status)


def make_dims(batch, seqlen, nheads, headdim, dstate, ngroups=1, chunk=256, dtype=F32) -> Dims:
    return Dims(int(batch), int(seqlen), int(nheads), int(headdim), int(dstate), int(ngroups),
                int(chunk), int(dtype))


def _p(t):
    return None if t is None else _vp(t.data_ptr())


def _stream():
    return _vp(torch.cuda.current_stream().cuda_stream)


def _need(t, name, shape, dtype, dev):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != dev:
        raise ValueError(f"{name} is on {t.device}, expected {dev}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _forward_dims(x, dt, A, B, C, D, init, chunk):
    if x.dim() != 4 or B.dim() != 4:
        raise ValueError("x must be [b, L, H, P] and B, C [b, L, G, N]")
    if x.dtype not in _DT:
        raise ValueError(f"unsupported dtype {x.dtype}")
    if x.device.type != "cuda":
        raise ValueError("inputs must be on a HIP device")
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    dev = x.device
    _need(x, "x", (b, L, H, P), x.dtype, dev)
    _need(dt, "dt", (b, L, H), x.dtype, dev)
    _need(A, "A", (H,), torch.float32, dev)
    _need(B, "B", (b, L, G, N), x.dtype, dev)
    _need(C, "C", (b, L, G, N), x.dtype, dev)
    if D is not None:
        _need(D, "D", (H,), torch.float32, dev)
    if init is not None:
        _need(init, "init_state", (b, H, P, N), torch.float32, dev)
    return make_dims(b, L, H, P, N, G, chunk, _DT[x.dtype])


def make_options(A, dt_bias=None, dt_softplus=False, dt_limit=None, input_scale="none"):
    """DtOptions for the keyword arguments of forward / decode_step, or None
    when they are all at their defaults (the plain map).  dt_limit: (lo, hi)
    clamp of the step after softplus."""
    if input_scale not in SCALES:
        raise ValueError(f"input_scale must be one of {tuple(SCALES)}")
    lo, hi = (0.0, 0.0) if dt_limit is None else (float(dt_limit[0]), float(dt_limit[1]))
    if dt_bias is None and not dt_softplus and not hi > lo and input_scale == "none":
        return None
    if dt_bias is not None:
        _need(dt_bias, "dt_bias", A.shape, torch.float32, A.device)
    return DtOptions(_p(dt_bias), int(bool(dt_softplus)), lo, hi, SCALES[input_scale])


def workspace_bytes(dims: Dims) -> int:
    return int(lib.ssd_forward_workspace_bytes(ctypes.byref(dims)))


def forward(x, dt, A, B, C, D=None, init_state=None, chunk: int = 256, *, staged: bool = False,
            y=None, final_state=None, workspace=None, want_final: bool = True, dt_bias=None,
            dt_softplus: bool = False, dt_limit=None, input_scale: str = "none"):
    """Layer forward (chunked algorithm).  Returns (y, final_state).

    ``y`` / ``final_state`` / ``workspace`` may be preallocated (the
    workspace as a uint8 CUDA tensor of at least ``workspace_bytes``);
    ``final_state`` may be ``init_state`` itself for an in-place carry.
    ``dt_bias`` / ``dt_softplus`` / ``dt_limit`` / ``input_scale`` select the
    step-size preprocessing and input scaling of ssd_forward_ex.
    """
    opts = make_options(A, dt_bias, dt_softplus, dt_limit, input_scale)
    dims = _forward_dims(x, dt, A, B, C, D, init_state, chunk)
    b, L, H, P = x.shape
    N = B.shape[3]
    if y is None:
        y = torch.empty_like(x)
    else:
        _need(y, "y", x.shape, x.dtype, x.device)
    if final_state is None and want_final:
        final_state = torch.empty((b, H, P, N), dtype=torch.float32, device=x.device)
    elif final_state is not None:
        _need(final_state, "final_state", (b, H, P, N), torch.float32, x.device)
    nbytes = workspace_bytes(dims)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=x.device)
    args = (_p(x), _p(dt), _p(A), _p(B), _p(C), _p(D), _p(init_state), _p(y), _p(final_state),
            _p(workspace), workspace.numel(), _stream())
    if opts is None:
        fn = lib.ssd_forward_staged if staged else lib.ssd_forward
        _check(fn(ctypes.byref(dims), *args))
    else:
        fn = lib.ssd_forward_staged_ex if staged else lib.ssd_forward_ex
        _check(fn(ctypes.byref(dims), ctypes.byref(opts), *args))
    return y, final_state


NOALLOC_WORKSPACE_BYTES = 32 << 20  # SSD_NOALLOC_WORKSPACE_BYTES


def forward_noalloc(x, dt, A, B, C, D=None, init_state=None, chunk: int = 256, *, y=None, final_state=None,
                    want_final: bool = True):
    """ssd_forward_noalloc: the forward with the library's own fixed device
    workspace (no workspace argument, no allocation inside the library).
    Returns (y, final_state); ``y`` / ``final_state`` may be preallocated so
    that the call itself allocates nothing on the torch side either.
    """
    dims = _forward_dims(x, dt, A, B, C, D, init_state, chunk)
    b, L, H, P = x.shape
    N = B.shape[3]
    if y is None:
        y = torch.empty_like(x)
    else:
        _need(y, "y", x.shape, x.dtype, x.device)
    if final_state is None and want_final:
        final_state = torch.empty((b, H, P, N), dtype=torch.float32, device=x.device)
    elif final_state is not None:
        _need(final_state, "final_state", (b, H, P, N), torch.float32, x.device)
    _check(lib.ssd_forward_noalloc(ctypes.byref(dims), _p(x), _p(dt), _p(A), _p(B), _p(C), _p(D),
                                   _p(init_state), _p(y), _p(final_state), _stream()))
    return y, final_state


def backward_workspace_bytes(dims: Dims) -> int:
    return int(lib.ssd_backward_workspace_bytes(ctypes.byref(dims)))


def backward(x, dt, A, B, C, dy, D=None, init_state=None, dfinal_state=None, chunk: int = 256, *,
             out=None, workspace=None, want_dD: bool = True, want_dinit: bool = True):
    """Gradient of sum(dy * y) + sum(dfinal_state * final_state) for the
    forward on the same inputs.  Returns a dict with dx, ddt, dA, dB, dC and
    (when wanted) dD and dinit (dx, ddt, dB, dC in the input dtype; dA, dD,
    dinit float32).  ``out`` may hold preallocated outputs under those names.
    """
    dims = _forward_dims(x, dt, A, B, C, D, init_state, chunk)
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    dev = x.device
    _need(dy, "dy", x.shape, x.dtype, dev)
    if dfinal_state is not None:
        _need(dfinal_state, "dfinal_state", (b, H, P, N), torch.float32, dev)
    shapes = {"dx": (x.shape, x.dtype), "ddt": (dt.shape, x.dtype), "dA": ((H,), torch.float32),
              "dB": (B.shape, x.dtype), "dC": (C.shape, x.dtype)}
    if want_dD:
        shapes["dD"] = ((H,), torch.float32)
    if want_dinit:
        shapes["dinit"] = ((b, H, P, N), torch.float32)
    out = dict(out or {})
    for k, (shp, dty) in shapes.items():
        if k in out:
            _need(out[k], k, shp, dty, dev)
        else:
            out[k] = torch.empty(tuple(shp), dtype=dty, device=dev)
    nbytes = backward_workspace_bytes(dims)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    _check(lib.ssd_backward(ctypes.byref(dims), _p(x), _p(dt), _p(A), _p(B), _p(C), _p(D),
                            _p(init_state), _p(dy), _p(dfinal_state), _p(out["dx"]), _p(out["ddt"]),
                            _p(out["dA"]), _p(out["dB"]), _p(out["dC"]), _p(out.get("dD")),
                            _p(out.get("dinit")), _p(workspace), workspace.numel(), _stream()))
    return out


SCAN_ALGOS = {"auto": 0, "segments": 1, "rows": 2}


class ScanDims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64), ("channels", ctypes.c_int64),
                ("dstate", ctypes.c_int64), ("ngroups", ctypes.c_int64), ("dtype", ctypes.c_int32),
                ("algo", ctypes.c_int32)]


def selective_scan(x, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus: bool = False,
                   init_state=None, *, y=None, final_state=None, want_final: bool = True, workspace=None,
                   algo: str = "auto"):
    """The selective (Mamba-1) scan, ssd_selective_scan.  x, delta, z
    [b, L, Dch]; A [Dch, N] float32; B, C [b, L, G, N] (or [b, L, N]); D,
    delta_bias [Dch] float32; init_state [b, Dch, N] float32.  algo: "auto",
    "segments" or "rows" (N = 16 only).  Returns (y, final_state)."""
    if x.dim() != 3 or x.dtype not in _DT:
        raise ValueError("x must be [b, L, channels] float32 / bfloat16")
    if B.dim() == 3:
        B, C = B.unsqueeze(2), C.unsqueeze(2)
    b, L, Dch = x.shape
    G, N = B.shape[2], B.shape[3]
    dev = x.device
    _need(x, "x", (b, L, Dch), x.dtype, dev)
    _need(delta, "delta", (b, L, Dch), x.dtype, dev)
    _need(A, "A", (Dch, N), torch.float32, dev)
    _need(B, "B", (b, L, G, N), x.dtype, dev)
    _need(C, "C", (b, L, G, N), x.dtype, dev)
    for t, nm in ((D, "D"), (delta_bias, "delta_bias")):
        if t is not None:
            _need(t, nm, (Dch,), torch.float32, dev)
    if z is not None:
        _need(z, "z", (b, L, Dch), x.dtype, dev)
    if init_state is not None:
        _need(init_state, "init_state", (b, Dch, N), torch.float32, dev)
    dims = ScanDims(b, L, Dch, N, G, _DT[x.dtype], SCAN_ALGOS[algo])
    if y is None:
        y = torch.empty_like(x)
    if final_state is None and want_final:
        final_state = torch.empty((b, Dch, N), dtype=torch.float32, device=dev)
    nbytes = int(lib.ssd_selective_scan_workspace_bytes(ctypes.byref(dims)))
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    _check(lib.ssd_selective_scan(ctypes.byref(dims), _p(x), _p(delta), _p(A), _p(B), _p(C), _p(D), _p(z),
                                  _p(delta_bias), int(bool(delta_softplus)), _p(init_state), _p(y),
                                  _p(final_state), _p(workspace), workspace.numel(), _stream()))
    return y, final_state


def gated_rmsnorm(y, z, weight, norm_groups: int = 1, eps: float = 1e-5, out=None):
    """out = RMSNorm(y * silu(z)) * weight per token over its H * P channels
    (norm_groups equal groups).  y, z [b, L, H, P] (or [b, H, P] for one
    token), weight [H * P] float32.  out may be y (in place)."""
    if y.dim() == 3:
        y4, z4 = y.unsqueeze(1), z.unsqueeze(1)
    else:
        y4, z4 = y, z
    if y4.dim() != 4 or y.dtype not in _DT:
        raise ValueError("y must be [b, L, H, P] or [b, H, P] float32 / bfloat16")
    b, L, H, P = y4.shape
    _need(z, "z", y.shape, y.dtype, y.device)
    _need(weight, "weight", (H * P,), torch.float32, y.device)
    _need(y, "y", y.shape, y.dtype, y.device)
    if out is None:
        out = torch.empty_like(y)
    else:
        _need(out, "out", y.shape, y.dtype, y.device)
    dims = make_dims(b, L, H, P, 16, 1, 16, _DT[y.dtype])
    _check(lib.ssd_gated_rmsnorm(ctypes.byref(dims), int(norm_groups), float(eps), _p(y), _p(z), _p(weight),
                                 _p(out), _stream()))
    return out


def decode_step(state, x, dt, A, B, C, D=None, y=None, *, dt_bias=None, dt_softplus: bool = False,
                dt_limit=None, input_scale: str = "none"):
    """One recurrent step; ``state`` [b, H, P, N] float32 is updated in place.

    x [b, H, P], dt [b, H], B, C [b, G, N].  Returns y [b, H, P].  The
    step-size keywords are those of forward (ssd_decode_step_ex)."""
    if x.dim() != 3 or B.dim() != 3:
        raise ValueError("x must be [b, H, P] and B, C [b, G, N]")
    if x.dtype not in _DT:
        raise ValueError(f"unsupported dtype {x.dtype}")
    b, H, P = x.shape
    G, N = B.shape[1], B.shape[2]
    dev = x.device
    _need(state, "state", (b, H, P, N), torch.float32, dev)
    _need(x, "x", (b, H, P), x.dtype, dev)
    _need(dt, "dt", (b, H), x.dtype, dev)
    _need(A, "A", (H,), torch.float32, dev)
    _need(B, "B", (b, G, N), x.dtype, dev)
    _need(C, "C", (b, G, N), x.dtype, dev)
    if D is not None:
        _need(D, "D", (H,), torch.float32, dev)
    if y is None:
        y = torch.empty_like(x)
    dims = make_dims(b, 1, H, P, N, G, 16, _DT[x.dtype])
    opts = make_options(A, dt_bias, dt_softplus, dt_limit, input_scale)
    args = (_p(state), _p(x), _p(dt), _p(A), _p(B), _p(C), _p(D), _p(y), _stream())
    if opts is None:
        _check(lib.ssd_decode_step(ctypes.byref(dims), *args))
    else:
        _check(lib.ssd_decode_step_ex(ctypes.byref(dims), ctypes.byref(opts), *args))
    return y


# ---------------------------------------------------------------- the steps
def _nc(L, Q):
    return (L + Q - 1) // Q


def chunk_cumsum(dt, A, chunk: int):
    """cs [b, H, nc, chunk] float32 (decay prefix inside each chunk)."""
    b, L, H = dt.shape
    dims = make_dims(b, L, H, 16, 16, 1, chunk, _DT[dt.dtype])
    cs = torch.empty((b, H, _nc(L, chunk), chunk), dtype=torch.float32, device=dt.device)
    _check(lib.ssd_chunk_cumsum(ctypes.byref(dims), _p(dt.contiguous()), _p(A), _p(cs), _stream()))
    return cs


def chunk_cb(B, C, chunk: int, nheads: int | None = None):
    """cb [b, nc, G, chunk, chunk] in B's dtype (lower tiles written)."""
    b, L, G, N = B.shape
    H = nheads or G
    dims = make_dims(b, L, H, 16, N, G, chunk, _DT[B.dtype])
    cb = torch.zeros((b, _nc(L, chunk), G, chunk, chunk), dtype=B.dtype, device=B.device)
    _check(lib.ssd_chunk_cb(ctypes.byref(dims), _p(B), _p(C), _p(cb), _stream()))
    return cb


def chunk_state(x, B, cs, chunk: int):
    """S [b, nc, H, P, N] float32 (each chunk's end state from zero)."""
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    dims = make_dims(b, L, H, P, N, G, chunk, _DT[x.dtype])
    S = torch.empty((b, _nc(L, chunk), H, P, N), dtype=torch.float32, device=x.device)
    _check(lib.ssd_chunk_state(ctypes.byref(dims), _p(x), _p(B), _p(cs), _p(S), _stream()))
    return S


def state_passing(S, cs, L: int, chunk: int, init_state=None, final_state=None):
    """In place: S -> hprev (state entering each chunk).  Returns (S, final)."""
    b, nc, H, P, N = S.shape
    dims = make_dims(b, L, H, P, N, 1, chunk, F32)
    if final_state is None:
        final_state = torch.empty((b, H, P, N), dtype=torch.float32, device=S.device)
    _check(lib.ssd_state_passing(ctypes.byref(dims), _p(S), _p(cs), _p(init_state), _p(final_state),
                                 _stream()))
    return S, final_state


def chunk_scan(x, C, cb, cs, hprev, D, chunk: int):
    """y: intra-chunk masked product + exp(cs) hprev C + D x."""
    b, L, H, P = x.shape
    G, N = C.shape[2], C.shape[3]
    dims = make_dims(b, L, H, P, N, G, chunk, _DT[x.dtype])
    y = torch.empty_like(x)
    _check(lib.ssd_chunk_scan(ctypes.byref(dims), _p(x), _p(C), _p(cb), _p(cs), _p(hprev), _p(D),
                              _p(y), _stream()))
    return y
