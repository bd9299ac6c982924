"""The scan pins must reject plausible mistakes planted in a copy of
selective_scan.c (the committed oracle is never modified)."""
import ctypes
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle
from test_oracle_scan_pins import case, page_loop, rel

SRC = os.path.join(os.path.dirname(oracle.__file__), "selective_scan.c")
MUTATIONS = {
    "decay_after_write": ("h[n] = exp(dl * A[d * N + n]) * h[n] + dl * Bt[n] * xv;",
                          "h[n] = exp(dl * A[d * N + n]) * (h[n] + dl * Bt[n] * xv);"),
    "no_step_on_B": ("+ dl * Bt[n] * xv;", "+ Bt[n] * xv;"),
    "read_before_update": ("h[n] = exp(dl * A[d * N + n]) * h[n] + dl * Bt[n] * xv;\n                acc += Ct[n] * h[n];",
                           "acc += Ct[n] * h[n];\n                h[n] = exp(dl * A[d * N + n]) * h[n] + dl * Bt[n] * xv;"),
    "gate_sigmoid": ("out *= z[i] / (1.0 + exp(-z[i]));", "out *= 1.0 / (1.0 + exp(-z[i]));"),
    "A_transposed": ("exp(dl * A[d * N + n])", "exp(dl * A[n * Dch + d])"),
}


def _run(name, c, **kw):
    import tempfile
    old, new = MUTATIONS[name]
    text = open(SRC).read()
    assert old in text, name
    with tempfile.TemporaryDirectory() as tmp:
        src = os.path.join(tmp, "m.c")
        open(src, "w").write(text.replace(old, new))
        so = os.path.join(tmp, "m.so")
        subprocess.check_call(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-std=c11", src, "-o", so, "-lm"])
        lib = ctypes.CDLL(so)
        i64, dp = ctypes.c_int64, ctypes.c_void_p
        lib.ssd_oracle_selective_scan.argtypes = [i64] * 5 + [dp] * 8 + [i64] + [dp] * 3
        f = lambda a: None if a is None else np.ascontiguousarray(a, np.float64)
        x, dl, A, B, C = (f(c[k]) for k in ("x", "delta", "A", "B", "C"))
        D, z = f(kw.get("D")), f(kw.get("z"))
        b, L, Dch = x.shape
        G, N = B.shape[2], B.shape[3]
        y = np.empty((b, L, Dch))
        fin = np.empty((b, Dch, N))
        p = lambda a: None if a is None else a.ctypes.data_as(dp)
        lib.ssd_oracle_selective_scan(b, L, Dch, N, G, p(x), p(dl), p(A), p(B), p(C), p(D), p(z), None, 0, None,
                                      p(y), p(fin))
        return y


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_scan_pins_reject_mutant(name):
    rng = np.random.default_rng(9)
    c = case(rng, Dch=6, N=5)
    yr, _ = page_loop(c["x"], c["delta"], c["A"], c["B"][:, :, 0], c["C"][:, :, 0])
    caught = rel(_run(name, c), yr) > 1e-9
    z = rng.standard_normal(c["x"].shape)
    D = rng.standard_normal(6)
    cz = dict(c, B=np.zeros_like(c["B"]))
    caught = caught or not np.allclose(_run(name, cz, D=D, z=z), D * c["x"] * z / (1 + np.exp(-z)), atol=1e-12)
    assert caught, name
