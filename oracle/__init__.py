"""CPU oracle for the SSD layer -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports, links or calls anything here, and nothing
here imports the product path: the two share only the seeded input
generator (``ssd_inputs``), which holds none of the method's arithmetic.

Contents
--------
* ``forward`` / ``decode_step``: the float64 sequential recurrence, in plain C
  (``ssd_recurrence.c``), parallel over independent (batch, head) sequences.
* ``backward``: reverse-mode differentiation of that recurrence, step by
  step in reverse order (``ssd_backward.c``), float64.
* ``gated_rmsnorm``: the normalisation after the gate (numpy float64).
* ``selective_scan``: the Mamba-1 scan with a diagonal A per channel, its
  skip term and gate (``selective_scan.c``, float64).
* ``preprocess_dt`` / ``forward_ex`` / ``decode_step_ex``: the step size
  through bias, softplus and clamp, and the Euler or zero-order-hold input
  scale, ahead of the same recurrence (numpy float64).
* ``chunked``: float64 numpy versions of each step of the chunked algorithm
  (decay prefix, C B^T, intra-chunk masked product, chunk state, state
  passing, output combine) used to check the GPU's intermediates.

Every function is pinned by ``tests/test_oracle_pins.py`` against what the
pages fix: the printed four-token example, the quadratic (masked attention)
form, the closed forms for a = 1 and constant a, the rank bound, the split
call and chunk-size invariance.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssd_recurrence.c")
_SRC_BWD = os.path.join(_HERE, "ssd_backward.c")
_SRC_SCAN = os.path.join(_HERE, "selective_scan.c")
_LIB_PATH = os.path.join(_HERE, "_build", "libssd_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (plain -O2 + OpenMP, no fast-math)."""
    os.makedirs(os.path.dirname(_LIB_PATH), exist_ok=True)
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                               _SRC, _SRC_BWD, _SRC_SCAN, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        lib = ctypes.CDLL(_LIB_PATH)
        i64, dp = ctypes.c_int64, ctypes.c_void_p
        lib.ssd_oracle_forward.argtypes = [i64] * 6 + [dp] * 9 + [i64, dp]
        lib.ssd_oracle_forward.restype = ctypes.c_int
        lib.ssd_oracle_backward.argtypes = [i64] * 6 + [dp] * 16
        lib.ssd_oracle_backward.restype = ctypes.c_int
        lib.ssd_oracle_selective_scan.argtypes = [i64] * 5 + [dp] * 8 + [i64] + [dp] * 3
        lib.ssd_oracle_selective_scan.restype = ctypes.c_int
        lib.ssd_oracle_decode_step.argtypes = [i64] * 5 + [dp] * 8
        lib.ssd_oracle_decode_step.restype = ctypes.c_int
        lib.ssd_oracle_num_threads.restype = ctypes.c_int
        lib.ssd_oracle_set_num_threads.argtypes = [ctypes.c_int]
        _lib = lib
    return _lib


def num_threads() -> int:
    return _load().ssd_oracle_num_threads()


def set_num_threads(n: int) -> None:
    _load().ssd_oracle_set_num_threads(int(n))


def _f64(a):
    if a is None:
        return None
    if hasattr(a, "detach"):  # torch tensor -> exact float64
        import torch
        a = a.detach().to("cpu").to(torch.float64).numpy()
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def forward(x, dt, A, B, C, D=None, init=None, chunk: int = 0):
    """Sequential float64 recurrence.

    Shapes: x [b, L, H, P], dt [b, L, H], A [H], B, C [b, L, G, N], D [H] or
    None, init [b, H, P, N] or None.  Returns (y, final_state) and, when
    ``chunk`` > 0, also the state entering every chunk, [b, nc, H, P, N].
    """
    x, dt, A, B, C, D, init = (_f64(v) for v in (x, dt, A, B, C, D, init))
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    assert dt.shape == (b, L, H) and A.shape == (H,) and B.shape == (b, L, G, N)
    assert C.shape == B.shape and (D is None or D.shape == (H,))
    assert init is None or init.shape == (b, H, P, N)
    y = np.empty((b, L, H, P))
    final = np.empty((b, H, P, N))
    bnd = None
    if chunk > 0:
        nc = (L + chunk - 1) // chunk
        bnd = np.empty((b, nc, H, P, N))
    rc = _load().ssd_oracle_forward(b, L, H, P, N, G, _ptr(x), _ptr(dt), _ptr(A), _ptr(B),
                                     _ptr(C), _ptr(D), _ptr(init), _ptr(y), _ptr(final),
                                     int(chunk), _ptr(bnd))
    if rc != 0:
        raise ValueError("oracle: bad shape")
    return (y, final, bnd) if chunk > 0 else (y, final)


def backward(x, dt, A, B, C, D, init, dy, dfinal=None):
    """Gradient of the forward map by reverse-mode differentiation of the
    sequential recurrence (float64).

    With loss = sum(dy * y) + sum(dfinal * final_state), returns a dict with
    dx [b, L, H, P], ddt [b, L, H], dA [H], dB and dC [b, L, G, N], dD [H]
    (zero-filled when D is None) and dinit [b, H, P, N] (the gradient of the
    initial state, also when init is None, i.e. zero).
    """
    x, dt, A, B, C, D, init, dy, dfinal = (_f64(v) for v in (x, dt, A, B, C, D, init, dy, dfinal))
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    assert dy.shape == x.shape and (dfinal is None or dfinal.shape == (b, H, P, N))
    dx = np.empty_like(x)
    ddt = np.empty((b, L, H))
    dB_h = np.empty((b, L, H, N))
    dC_h = np.empty((b, L, H, N))
    dA_bh = np.empty((b, H))
    dD_bh = np.empty((b, H))
    dinit = np.empty((b, H, P, N))
    rc = _load().ssd_oracle_backward(b, L, H, P, N, G, _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C),
                                      _ptr(D), _ptr(init), _ptr(dy), _ptr(dfinal), _ptr(dx), _ptr(ddt),
                                      _ptr(dB_h), _ptr(dC_h), _ptr(dA_bh), _ptr(dD_bh), _ptr(dinit))
    if rc != 0:
        raise ValueError("oracle backward: bad shape or out of memory")
    hg = H // G
    return {"dx": dx, "ddt": ddt, "dA": dA_bh.sum(axis=0),
            "dB": dB_h.reshape(b, L, G, hg, N).sum(axis=3), "dC": dC_h.reshape(b, L, G, hg, N).sum(axis=3),
            "dD": dD_bh.sum(axis=0), "dinit": dinit}


SCALES = ("none", "euler", "zoh")


def preprocess_dt(dt, A, dt_bias=None, softplus=False, dt_min=0.0, dt_max=0.0, scale="none"):
    """The step size and input scale of one (step, head), float64.

    dt_eff = softplus(dt + dt_bias) when ``softplus`` (Mamba review, section
    3.1: the step size is a softplus of a linear map of the input, whose bias
    is dt_bias), else dt + dt_bias; then clamped to [dt_min, dt_max] when
    dt_max > dt_min.  The input scale s multiplies x in the state update:
      "none":  s = 1 (the SSD pages add B x with no step factor);
      "euler": s = dt_eff (Mamba review, section 3.3: B discretised as dt B);
      "zoh":   s = integral_0^dt_eff exp(u A) du = expm1(dt_eff A) / A, dt_eff
               when A = 0 (Mamba review, section 2.2; guide, equation (2)).
    dt [..., H], A [H].  Returns (dt_eff, s), both shaped like dt.
    """
    if scale not in SCALES:
        raise ValueError(f"scale must be one of {SCALES}")
    d = _f64(dt)
    A = _f64(A)
    if dt_bias is not None:
        d = d + _f64(dt_bias)
    if softplus:
        d = np.logaddexp(0.0, d)          # log(1 + e^d), without overflow
    if dt_max > dt_min:
        d = np.clip(d, dt_min, dt_max)
    if scale == "none":
        s = np.ones_like(d)
    elif scale == "euler":
        s = d.copy()
    else:
        Ab = np.broadcast_to(A, d.shape)
        with np.errstate(divide="ignore", invalid="ignore"):
            s = np.where(Ab != 0.0, np.expm1(d * Ab) / Ab, d)
    return d, s


def forward_ex(x, dt, A, B, C, D=None, init=None, dt_bias=None, softplus=False, dt_min=0.0,
               dt_max=0.0, scale="none", chunk: int = 0):
    """forward() with the step size preprocessed and the input scaled as in
    preprocess_dt: the recurrence runs on (s x, dt_eff), and the skip term
    uses the raw input, y += D x (Mamba review, section 3.4: D is a separate
    block parameter)."""
    d, s_ = preprocess_dt(dt, A, dt_bias, softplus, dt_min, dt_max, scale)
    x = _f64(x)
    out = forward(s_[..., None] * x, d, A, B, C, None, init, chunk=chunk)
    y = out[0]
    if D is not None:
        y = y + _f64(D)[None, None, :, None] * x
    return (y,) + tuple(out[1:])


def decode_step_ex(state, x, dt, A, B, C, D=None, dt_bias=None, softplus=False, dt_min=0.0,
                   dt_max=0.0, scale="none"):
    """decode_step() with preprocess_dt applied to the step's dt [b, H] and
    the skip term on the raw input."""
    d, s_ = preprocess_dt(dt, A, dt_bias, softplus, dt_min, dt_max, scale)
    x = _f64(x)
    y, state = decode_step(state, s_[..., None] * x, d, A, B, C, None)
    if D is not None:
        y = y + _f64(D)[None, :, None] * x
    return y, state


def selective_scan(x, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=False,
                   init=None):
    """The selective (Mamba-1) scan in float64 (``selective_scan.c``).

    x, delta, z [b, L, Dch]; A [Dch, N]; B, C [b, L, G, N] (or [b, L, N] for
    one group); D, delta_bias [Dch]; init [b, Dch, N].  Returns (y, final).
    """
    x, delta, A, B, C, D, z, delta_bias, init = (_f64(v) for v in (x, delta, A, B, C, D, z, delta_bias, init))
    if B.ndim == 3:
        B, C = B[:, :, None, :], C[:, :, None, :]
    b, L, Dch = x.shape
    G, N = B.shape[2], B.shape[3]
    assert A.shape == (Dch, N) and delta.shape == x.shape and C.shape == B.shape
    y = np.empty((b, L, Dch))
    final = np.empty((b, Dch, N))
    rc = _load().ssd_oracle_selective_scan(b, L, Dch, N, G, _ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C),
                                           _ptr(D), _ptr(z), _ptr(delta_bias), int(bool(delta_softplus)),
                                           _ptr(init), _ptr(y), _ptr(final))
    if rc != 0:
        raise ValueError("oracle selective_scan: bad shape")
    return y, final


def gated_rmsnorm(y, z, weight, norm_groups: int = 1, eps: float = 1e-5):
    """The normalisation after the gate, float64.

    The review page (section "Mamba-2 ブロック") adds one normalisation layer
    after the SSM output is multiplied by the gate and before the output
    projection; the Mamba review (section 3.4) gates with SiLU of a second
    projection z.  Reading (the kind of normalisation is not stated): per
    token, g = y * silu(z) over its H * P channels, split into norm_groups
    equal contiguous groups, each scaled to unit root mean square,
      out = g / sqrt(mean_group(g^2) + eps) * weight.
    y, z [..., H, P]; weight [H * P].  Returns out, shaped like y.
    """
    y, z, w = _f64(y), _f64(z), _f64(weight)
    shp = y.shape
    D = shp[-2] * shp[-1]
    if D % norm_groups:
        raise ValueError("norm_groups must divide H * P")
    g = y * (z / (1.0 + np.exp(-z)))                     # silu(z) = z sigmoid(z)
    g = g.reshape(-1, norm_groups, D // norm_groups)
    ms = np.mean(g * g, axis=-1, keepdims=True)
    out = g / np.sqrt(ms + eps) * w.reshape(1, norm_groups, D // norm_groups)
    return out.reshape(shp)


def decode_step(state, x, dt, A, B, C, D=None):
    """One recurrence step on a carried state.

    state [b, H, P, N] (float64, updated in place and returned), x [b, H, P],
    dt [b, H], B, C [b, G, N].  Returns (y [b, H, P], state).
    """
    assert isinstance(state, np.ndarray) and state.dtype == np.float64 and state.flags.c_contiguous
    x, dt, A, B, C, D = (_f64(v) for v in (x, dt, A, B, C, D))
    b, H, P, N = state.shape
    G = B.shape[1]
    y = np.empty((b, H, P))
    rc = _load().ssd_oracle_decode_step(b, H, P, N, G, _ptr(state), _ptr(x), _ptr(dt), _ptr(A),
                                         _ptr(B), _ptr(C), _ptr(D), _ptr(y))
    if rc != 0:
        raise ValueError("oracle: bad shape")
    return y, state
