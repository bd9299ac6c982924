"""Pins of the step-size preprocessing and input scaling in the oracle
(oracle.preprocess_dt, forward_ex, decode_step_ex).

None compares the oracle with a retyping of itself:
  * softplus against its identities and limits;
  * the zero-order-hold scale against numerical quadrature of its integral
    form (guide, equation (2)), including A = 0;
  * the whole zero-order-hold forward against a numerical solution of the
    continuous system h' = A h + x(t) B^T with the input held constant over
    each step and the readout at the step's end (Mamba review, section 2.2);
  * the Euler forward against our own transcription of the Mamba-1 scan
    (Mamba review, section 3.3, whose discretised B is dt B);
  * the bias and softplus through the inverse softplus; the clamp; the skip
    term on the raw input; decode against forward.
"""
import numpy as np
import pytest
from scipy.integrate import quad, solve_ivp

import oracle


def rel(a, r):
    a, r = np.asarray(a, np.float64), np.asarray(r, np.float64)
    return float(np.linalg.norm(a - r) / max(np.linalg.norm(r), 1e-300))


def test_softplus_identities():
    z = np.array([-40.0, -5.0, -0.3, 0.0, 0.7, 6.0, 60.0])
    sp = lambda v: oracle.preprocess_dt(v[None, :], np.zeros(len(v)), softplus=True)[0][0]
    s, sm = sp(z), sp(-z)
    assert abs(sp(np.array([0.0]))[0] - np.log(2.0)) < 1e-15
    assert np.allclose(s - sm, z, rtol=0, atol=1e-12)            # softplus(z) - softplus(-z) = z
    assert abs(s[0] / np.exp(-40.0) - 1) < 1e-12                 # e^z for very negative z
    assert s[-1] == 60.0
    assert np.all(np.diff(s) > 0)


@pytest.mark.parametrize("A", [-7.5, -1.0, -0.01, 0.0, 0.4])
@pytest.mark.parametrize("d", [1e-4, 0.05, 0.9, 3.0])
def test_zoh_scale_is_the_integral(A, d):
    _, s = oracle.preprocess_dt(np.array([[d]]), np.array([A]), scale="zoh")
    ref, _ = quad(lambda u: np.exp(u * A), 0.0, d, epsabs=0, epsrel=1e-13)
    assert abs(s[0, 0] - ref) <= 1e-12 * ref


def test_zoh_forward_solves_the_continuous_system():
    rng = np.random.default_rng(3)
    L, N, H = 6, 2, 2
    x = rng.standard_normal((1, L, H, 1))
    d = rng.uniform(0.05, 0.8, (1, L, H))
    A = np.array([-1.7, -0.4])
    B = rng.standard_normal((1, L, 1, N))
    C = rng.standard_normal((1, L, 1, N))
    D = np.array([0.3, -1.1])
    y, fin = oracle.forward_ex(x, d, A, B, C, D, scale="zoh")
    for h in range(H):
        state = np.zeros(N)
        for t in range(L):
            rhs = lambda _t, st, t=t: A[h] * st + x[0, t, h, 0] * B[0, t, 0]
            sol = solve_ivp(rhs, (0.0, d[0, t, h]), state, method="DOP853", rtol=1e-12, atol=1e-14)
            state = sol.y[:, -1]
            yt = state @ C[0, t, 0] + D[h] * x[0, t, h, 0]
            assert abs(yt - y[0, t, h, 0]) <= 1e-9 * max(1.0, abs(yt))
        assert np.allclose(state, fin[0, h, 0], rtol=1e-9, atol=1e-12)


def test_euler_forward_is_the_mamba1_scan():
    """Our transcription of the Mamba review's selective_scan loop (section
    3.3) with a per-channel A constant over the state index."""
    rng = np.random.default_rng(13)
    Bt, L, Dch, N = 2, 15, 3, 4
    x = rng.standard_normal((Bt, L, Dch))
    delta = np.exp(rng.uniform(-4, 0, (Bt, L, Dch)))
    Ad = -rng.uniform(0.5, 3, Dch)
    A = np.repeat(Ad[:, None], N, axis=1)
    Bm = rng.standard_normal((Bt, L, N))
    Cm = rng.standard_normal((Bt, L, N))
    ys = np.zeros((Bt, L, Dch))
    h = np.zeros((Bt, Dch, N))
    for t in range(L):
        h = np.exp(delta[:, t, :, None] * A[None]) * h + delta[:, t, :, None] * Bm[:, t, None, :] * x[:, t, :, None]
        ys[:, t] = (h * Cm[:, t, None, :]).sum(-1)
    y, _ = oracle.forward_ex(x[..., None], delta, Ad, Bm[:, :, None, :], Cm[:, :, None, :], scale="euler")
    assert rel(y[..., 0], ys) < 1e-12


def _case(rng, b=2, L=11, H=4, P=3, N=5, G=2):
    return dict(x=rng.standard_normal((b, L, H, P)), A=-rng.uniform(0.5, 3.0, H),
                B=rng.standard_normal((b, L, G, N)), C=rng.standard_normal((b, L, G, N)),
                D=rng.standard_normal(H), init=rng.standard_normal((b, H, P, N)))


@pytest.mark.parametrize("scale", oracle.SCALES)
def test_bias_and_softplus_through_the_inverse(scale):
    rng = np.random.default_rng(4)
    c = _case(rng)
    d0 = rng.uniform(0.01, 0.6, (2, 11, 4))
    bias = rng.standard_normal(4)
    raw = np.log(np.expm1(d0)) - bias                          # softplus(raw + bias) = d0
    y1, f1 = oracle.forward_ex(dt=raw, dt_bias=bias, softplus=True, scale=scale, **c)
    y2, f2 = oracle.forward_ex(dt=d0, scale=scale, **c)
    assert rel(y1, y2) < 1e-12 and rel(f1, f2) < 1e-12


def test_clamp():
    rng = np.random.default_rng(5)
    c = _case(rng)
    raw = rng.uniform(0.2, 0.9, (2, 11, 4))
    y1, _ = oracle.forward_ex(dt=raw, dt_min=0.0, dt_max=0.1, scale="zoh", **c)
    y2, _ = oracle.forward_ex(dt=np.full_like(raw, 0.1), scale="zoh", **c)
    assert rel(y1, y2) < 1e-14


@pytest.mark.parametrize("scale", oracle.SCALES)
def test_skip_term_uses_the_raw_input(scale):
    rng = np.random.default_rng(6)
    c = _case(rng)
    c["B"] = np.zeros_like(c["B"])
    c["init"] = None
    dt = rng.uniform(0.1, 0.5, (2, 11, 4))
    y, _ = oracle.forward_ex(dt=dt, scale=scale, **c)
    assert np.allclose(y, c["D"][None, None, :, None] * c["x"], rtol=0, atol=1e-15)


@pytest.mark.parametrize("scale", oracle.SCALES)
def test_decode_ex_equals_forward_ex(scale):
    rng = np.random.default_rng(7)
    c = _case(rng)
    raw = rng.standard_normal((2, 11, 4))
    bias = rng.standard_normal(4)
    kw = dict(dt_bias=bias, softplus=True, dt_min=0.01, dt_max=2.0, scale=scale)
    y, fin = oracle.forward_ex(dt=raw, **c, **kw)
    st = np.array(c["init"], dtype=np.float64, copy=True)
    for t in range(11):
        yt, st = oracle.decode_step_ex(st, c["x"][:, t], raw[:, t], c["A"], c["B"][:, t], c["C"][:, t], c["D"], **kw)
        assert rel(yt, y[:, t]) < 1e-12
    assert rel(st, fin) < 1e-12
