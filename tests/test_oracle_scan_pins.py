"""Pins of oracle.selective_scan (the Mamba-1 scan), none comparing it with
itself:
  * our numpy transcription of the Mamba review's selective_scan loop
    (section 3.3), with a general A [D, N];
  * the reduction to the SSD layer when A is constant over the state index
    (one channel per head, input dt x): the other C oracle;
  * the closed form of constant inputs (a geometric series);
  * the split call; the skip term and gate with B = 0; the step bias and
    softplus through the inverse softplus.
test_oracle_scan_mutations.py plants mistakes that these pins must reject.
"""
import numpy as np
import pytest

import oracle


def rel(a, r):
    a, r = np.asarray(a, np.float64), np.asarray(r, np.float64)
    return float(np.linalg.norm(a - r) / max(np.linalg.norm(r), 1e-300))


def case(rng, b=2, L=23, Dch=6, N=5, G=1):
    return dict(x=rng.standard_normal((b, L, Dch)), delta=np.exp(rng.uniform(-4, 0, (b, L, Dch))),
                A=-rng.uniform(0.2, 4.0, (Dch, N)), B=rng.standard_normal((b, L, G, N)),
                C=rng.standard_normal((b, L, G, N)))


def page_loop(x, delta, A, B, C):
    """The review's loop: deltaA = exp(delta A), deltaB = delta B, h = deltaA h + deltaB x, y = sum h C."""
    Bt, L, Dc = x.shape
    h = np.zeros((Bt, Dc, A.shape[1]))
    ys = np.zeros((Bt, L, Dc))
    for t in range(L):
        dA = np.exp(delta[:, t, :, None] * A[None])
        dB = delta[:, t, :, None] * B[:, t, None, :]
        h = dA * h + dB * x[:, t, :, None]
        ys[:, t] = (h * C[:, t, None, :]).sum(-1)
    return ys, h


def test_matches_the_page_loop():
    rng = np.random.default_rng(1)
    c = case(rng)
    y, fin = oracle.selective_scan(c["x"], c["delta"], c["A"], c["B"][:, :, 0], c["C"][:, :, 0])
    yr, hr = page_loop(c["x"], c["delta"], c["A"], c["B"][:, :, 0], c["C"][:, :, 0])
    assert rel(y, yr) < 1e-12 and rel(fin, hr) < 1e-12


@pytest.mark.parametrize("G", [1, 3])
def test_reduces_to_the_ssd_layer(G):
    rng = np.random.default_rng(2)
    c = case(rng, G=G)
    Ad = -rng.uniform(0.2, 4.0, 6)
    A = np.repeat(Ad[:, None], 5, axis=1)
    D = rng.standard_normal(6)
    init = rng.standard_normal((2, 6, 5))
    y, fin = oracle.selective_scan(c["x"], c["delta"], A, c["B"], c["C"], D=D, init=init)
    ys, fs = oracle.forward((c["delta"] * c["x"])[..., None], c["delta"], Ad, c["B"], c["C"], None,
                            init[:, :, None, :])
    assert rel(y, ys[..., 0] + D * c["x"]) < 1e-12
    assert rel(fin, fs[:, :, 0]) < 1e-12


def test_constant_inputs_geometric_series():
    L, N = 40, 3
    dl, a_, xv = 0.3, -1.2, 0.7
    Bv, Cv = np.array([0.5, -1.0, 2.0]), np.array([1.5, 0.25, -0.75])
    x = np.full((1, L, 1), xv)
    delta = np.full((1, L, 1), dl)
    A = np.full((1, N), a_)
    B = np.broadcast_to(Bv, (1, L, 1, N)).copy()
    C = np.broadcast_to(Cv, (1, L, 1, N)).copy()
    y, _ = oracle.selective_scan(x, delta, A, B, C)
    q = np.exp(dl * a_)
    t = np.arange(L)
    ref = (1 - q ** (t + 1)) / (1 - q) * dl * xv * (Bv @ Cv)
    assert np.allclose(y[0, :, 0], ref, rtol=1e-12)


def test_split_call_bitwise():
    rng = np.random.default_rng(3)
    c = case(rng, L=30)
    y, fin = oracle.selective_scan(**c)
    y1, f1 = oracle.selective_scan(**{k: (v[:, :13] if k in ("x", "delta", "B", "C") else v) for k, v in c.items()})
    y2, f2 = oracle.selective_scan(**{k: (v[:, 13:] if k in ("x", "delta", "B", "C") else v) for k, v in c.items()},
                                   init=f1)
    assert np.array_equal(np.concatenate([y1, y2], 1), y) and np.array_equal(f2, fin)


def test_skip_and_gate():
    rng = np.random.default_rng(4)
    c = case(rng)
    c["B"] = np.zeros_like(c["B"])
    D = rng.standard_normal(6)
    z = rng.standard_normal(c["x"].shape)
    y, _ = oracle.selective_scan(**c, D=D, z=z)
    assert np.allclose(y, D * c["x"] * z / (1 + np.exp(-z)), rtol=0, atol=1e-14)


def test_delta_bias_and_softplus_through_the_inverse():
    rng = np.random.default_rng(5)
    c = case(rng)
    bias = rng.standard_normal(6)
    raw = np.log(np.expm1(c["delta"])) - bias
    y1, f1 = oracle.selective_scan(**dict(c, delta=raw), delta_bias=bias, delta_softplus=True)
    y2, f2 = oracle.selective_scan(**c)
    assert rel(y1, y2) < 1e-12 and rel(f1, f2) < 1e-12
