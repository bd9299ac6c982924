"""The pins must catch plausible mistakes in the oracle.

Each case copies the oracle's C source to a temporary directory, plants one
mistake there (a dropped term, a wrong sign, a swapped operand, a wrong
index), builds it, and checks that the quadratic-form pin or the worked
example rejects it.  The committed oracle is never modified.
"""
import ctypes
import json
import math
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle
from test_oracle_pins import quadratic_form, rand_case, rel

SRC = os.path.join(os.path.dirname(oracle.__file__), "ssd_recurrence.c")

MUTATIONS = {
    "no_decay": ("hp[n] = a * hp[n] + xt[p] * Bt[n];", "hp[n] = hp[n] + xt[p] * Bt[n];"),
    "decay_after_write": ("hp[n] = a * hp[n] + xt[p] * Bt[n];", "hp[n] = a * (hp[n] + xt[p] * Bt[n]);"),
    "no_skip": ("yt[p] = acc + Dh * xt[p];", "yt[p] = acc;"),
    "decay_sign": ("exp(dt[(b * L + t) * H + h] * Ah)", "exp(-dt[(b * L + t) * H + h] * Ah)"),
    "swap_B_C": ("acc += hp[n] * Ct[n];", "acc += hp[n] * Bt[n];"),
    "group_map": ("const int64_t g = h / (H / G);", "const int64_t g = h % G;"),
    "ignore_init": ("memcpy(state, init + bh * P * N, sizeof(double) * P * N);",
                    "memset(state, 0, sizeof(double) * P * N);"),
    "read_before_update": ("hp[n] = a * hp[n] + xt[p] * Bt[n];\n                acc += hp[n] * Ct[n];",
                           "acc += hp[n] * Ct[n];\n                hp[n] = a * hp[n] + xt[p] * Bt[n];"),
}


def _build_mutant(tmp_path, name):
    old, new = MUTATIONS[name]
    text = open(SRC).read()
    assert old in text, name
    src = tmp_path / f"{name}.c"
    src.write_text(text.replace(old, new))
    so = tmp_path / f"{name}.so"
    subprocess.check_call(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-std=c11", str(src),
                           "-o", str(so), "-lm"])
    lib = ctypes.CDLL(str(so))
    i64, dp = ctypes.c_int64, ctypes.c_void_p
    lib.ssd_oracle_forward.argtypes = [i64] * 6 + [dp] * 9 + [i64, dp]
    return lib


def _run(lib, c):
    f = lambda a: None if a is None else np.ascontiguousarray(a, np.float64)
    x, dt, A, B, C, D, init = (f(c[k]) for k in ("x", "dt", "A", "B", "C", "D", "init"))
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    y = np.empty((b, L, H, P))
    fin = np.empty((b, H, P, N))
    p = lambda a: None if a is None else a.ctypes.data_as(ctypes.c_void_p)
    lib.ssd_oracle_forward(b, L, H, P, N, G, p(x), p(dt), p(A), p(B), p(C), p(D), p(init),
                           p(y), p(fin), 0, None)
    return y, fin


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_reject_mutant(tmp_path, name):
    lib = _build_mutant(tmp_path, name)
    caught = []
    c = rand_case(np.random.default_rng(0), G=2)
    y, fin = _run(lib, c)
    yq, fq = quadratic_form(**c)
    caught.append(rel(y, yq) > 1e-6 or rel(fin, fq) > 1e-6)
    ex = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")))
    a = np.array(ex["a"])
    y2, _ = _run(lib, dict(x=np.array(ex["x"]).reshape(1, 4, 1, 1), dt=(-np.log(a)).reshape(1, 4, 1),
                           A=np.array([-1.0]), B=np.array(ex["B"], float).reshape(1, 4, 1, 2),
                           C=np.array(ex["C"], float).reshape(1, 4, 1, 2), D=None, init=None))
    caught.append(not np.allclose(y2.ravel(), ex["y_printed"], atol=1e-9))
    assert any(caught), f"mutation {name} slipped through every pin"
