"""The backward pins must catch plausible mistakes in the backward oracle.

Each case copies ssd_backward.c to a temporary directory, plants one mistake
(a dropped factor, a term taken at the wrong time step, a missing decay, a
wrong checkpoint), builds it alone, and checks that the autograd pin of the
quadratic form or the directional finite difference rejects it.  The
committed oracle is never modified.
"""
import ctypes
import os
import shutil
import subprocess

import numpy as np
import pytest
import torch

import oracle
from test_oracle_backward_pins import GRAD_OF, case, loss, quadratic_form_torch, rel

SRC = os.path.join(os.path.dirname(oracle.__file__), "ssd_backward.c")

MUTATIONS = {
    "no_adjoint_decay": ("for (int64_t i = 0; i < PN; ++i) gst[i] *= a;", ""),
    "ddt_without_a": ("ddt[(b * L + t) * H + h] = da * a * Ah;", "ddt[(b * L + t) * H + h] = da * Ah;"),
    "dA_without_dt": ("dA += da * a * dtt;", "dA += da * a;"),
    "da_uses_h_t": ("da += gst[i] * hprev[i];", "da += gst[i] * ht[i];"),
    "dC_uses_h_prev": ("acc += ht[p * N + n] * dyt[p];", "acc += hprev[p * N + n] * dyt[p];"),
    "dx_no_skip": ("dxt[p] = acc + Dh * dyt[p];", "dxt[p] = acc;"),
    "dx_uses_C": ("acc += gst[p * N + n] * Bt[n];", "acc += gst[p * N + n] * Ct[n];"),
    "wrong_checkpoint": ("memcpy(state, ck + s * PN, sizeof(double) * PN);",
                         "memcpy(state, ck + (s > 0 ? s - 1 : 0) * PN, sizeof(double) * PN);"),
    "dfinal_ignored": ("gst[i] = dfinal ? dfinal[(b * H + h) * PN + i] : 0.0;", "gst[i] = 0.0;"),
    "group_map": ("const int64_t g = h / (H / G);", "const int64_t g = h % G;"),
}


def _build_mutant(tmp_path, name):
    old, new = MUTATIONS.get(name, ("", ""))
    text = open(SRC).read()
    assert old in text, name
    src = tmp_path / f"{name}.c"
    src.write_text(text.replace(old, new) if old else text)
    so = tmp_path / f"{name}.so"
    subprocess.check_call(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-std=c11", str(src),
                           "-o", str(so), "-lm"])
    lib = ctypes.CDLL(str(so))
    lib.ssd_oracle_backward.argtypes = [ctypes.c_int64] * 6 + [ctypes.c_void_p] * 16
    return lib


def _run(lib, c, dy, df):
    f = lambda a: None if a is None else np.ascontiguousarray(a, np.float64)
    x, dt, A, B, C, D, init = (f(c[k]) for k in ("x", "dt", "A", "B", "C", "D", "init"))
    dy, df = f(dy), f(df)
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    out = dict(dx=np.empty_like(x), ddt=np.empty((b, L, H)), dB_h=np.empty((b, L, H, N)),
               dC_h=np.empty((b, L, H, N)), dA_bh=np.empty((b, H)), dD_bh=np.empty((b, H)),
               dinit=np.empty((b, H, P, N)))
    p = lambda a: None if a is None else a.ctypes.data_as(ctypes.c_void_p)
    lib.ssd_oracle_backward(b, L, H, P, N, G, p(x), p(dt), p(A), p(B), p(C), p(D), p(init), p(dy), p(df),
                            *(p(out[k]) for k in ("dx", "ddt", "dB_h", "dC_h", "dA_bh", "dD_bh", "dinit")))
    hg = H // G
    return {"dx": out["dx"], "ddt": out["ddt"], "dA": out["dA_bh"].sum(0), "dD": out["dD_bh"].sum(0),
            "dB": out["dB_h"].reshape(b, L, G, hg, N).sum(3), "dC": out["dC_h"].reshape(b, L, G, hg, N).sum(3),
            "dinit": out["dinit"]}


def _autograd(c, dy, df):
    t = {k: torch.tensor(v, dtype=torch.float64, requires_grad=True) for k, v in c.items()}
    y, fin = quadratic_form_torch(**t)
    ((y * torch.tensor(dy)).sum() + (fin * torch.tensor(df)).sum()).backward()
    return {GRAD_OF[k]: t[k].grad.numpy() for k in t}


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_backward_pins_reject_mutant(tmp_path, name):
    lib = _build_mutant(tmp_path, name)
    rng = np.random.default_rng(20)
    # L = 80 crosses one 64-step checkpoint boundary; G = 2 with 4 heads
    c, dy, df = case(rng, b=1, L=80, H=4, P=2, N=3, G=2)
    got = _run(lib, c, dy, df)
    ref = _autograd(c, dy, df)
    caught = any(rel(got[k], ref[k]) > 1e-6 for k in ref)
    v = rng.standard_normal(c["dt"].shape)
    eps = 1e-6
    cp, cm = dict(c), dict(c)
    cp["dt"], cm["dt"] = c["dt"] + eps * v, c["dt"] - eps * v
    fd = (loss(cp, dy, df) - loss(cm, dy, df)) / (2 * eps)
    caught = caught or abs(fd - float(np.sum(got["ddt"] * v))) > 1e-6 * max(1.0, abs(fd))
    assert caught, f"mutation {name} slipped through every backward pin"


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_unmutated_copy_passes(tmp_path):
    """Control: the same build and check on the unmodified source accepts it."""
    lib = _build_mutant(tmp_path, "control")
    rng = np.random.default_rng(20)
    c, dy, df = case(rng, b=1, L=80, H=4, P=2, N=3, G=2)
    got = _run(lib, c, dy, df)
    ref = _autograd(c, dy, df)
    assert all(rel(got[k], ref[k]) < 1e-10 for k in ref)
