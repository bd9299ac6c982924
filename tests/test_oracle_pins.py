"""Pins of the CPU oracle against what the pages and the mathematics fix.

Nothing here compares the oracle with itself: each test checks it against a
value printed on a page, a closed form, a different algorithm for the same
map (the quadratic masked form, the chunked decomposition, a transcription
of the Mamba-1 scan), or an invariant that a plausible mistake (a dropped
term, a wrong sign or index, a transposed operand) would break.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import chunked

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rel(a, r):
    a, r = np.asarray(a, np.float64), np.asarray(r, np.float64)
    return float(np.linalg.norm((a - r).ravel()) / max(np.linalg.norm(r.ravel()), 1e-30))


def rand_case(rng, b=2, L=13, H=4, P=3, N=5, G=1, with_D=True, with_init=True):
    x = rng.standard_normal((b, L, H, P))
    B = rng.standard_normal((b, L, G, N)) / math.sqrt(N)
    C = rng.standard_normal((b, L, G, N)) / math.sqrt(N)
    dt = np.exp(rng.uniform(math.log(1e-2), math.log(1.0), (b, L, H)))
    A = -rng.uniform(0.5, 4.0, H)
    D = rng.standard_normal(H) if with_D else None
    init = rng.standard_normal((b, H, P, N)) if with_init else None
    return dict(x=x, dt=dt, A=A, B=B, C=C, D=D, init=init)


# ---------------------------------------------------------------- worked example
@pytest.fixture(scope="module")
def example():
    with open(os.path.join(GOLDEN, "worked_example.json")) as f:
        ex = json.load(f)
    a = np.array(ex["a"])
    case = dict(
        x=np.array(ex["x"]).reshape(1, 4, 1, 1),
        dt=(-np.log(a)).reshape(1, 4, 1),          # with A = -1: exp(dt * A) = a
        A=np.array([-1.0]),
        B=np.array(ex["B"], float).reshape(1, 4, 1, 2),
        C=np.array(ex["C"], float).reshape(1, 4, 1, 2),
    )
    return ex, case


def test_worked_example_recurrence(example):
    ex, c = example
    y, final = oracle.forward(**c)
    np.testing.assert_allclose(y.ravel(), ex["y_printed"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(final.ravel(), ex["final_state_derived"], rtol=0, atol=1e-12)


def test_worked_example_mask(example):
    ex, c = example
    cs = chunked.chunk_cumsum(c["dt"], c["A"], 4)[0, 0, 0]
    Lm = np.tril(np.exp(cs[:, None] - cs[None, :]))
    np.testing.assert_allclose(Lm, np.array(ex["L_printed"]), rtol=0, atol=1e-12)


@pytest.mark.parametrize("Q", [1, 2, 3, 4, 8])
def test_worked_example_chunked(example, Q):
    ex, c = example
    y, final, _ = chunked.forward_chunked(**c, Q=Q)
    np.testing.assert_allclose(y.ravel(), ex["y_printed"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(final.ravel(), ex["final_state_derived"], rtol=0, atol=1e-12)


def test_worked_example_intra_single_chunk(example):
    """One chunk, zero init: the masked product alone is the whole answer."""
    ex, c = example
    cs = chunked.chunk_cumsum(c["dt"], c["A"], 4)
    Gm = chunked.chunk_cb(c["C"], c["B"], 4)
    y = chunked.chunk_scan_intra(Gm, cs, c["x"], 4)
    np.testing.assert_allclose(y.ravel(), ex["y_printed"], rtol=0, atol=1e-12)


def test_worked_example_decode(example):
    ex, c = example
    state = np.zeros((1, 1, 1, 2))
    ys = []
    for t in range(4):
        y, state = oracle.decode_step(state, c["x"][:, t], c["dt"][:, t], c["A"], c["B"][:, t],
                                      c["C"][:, t])
        ys.append(float(y.ravel()[0]))
    np.testing.assert_allclose(ys, ex["y_printed"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(state.ravel(), ex["final_state_derived"], rtol=0, atol=1e-12)


# ---------------------------------------------------------------- quadratic form
def quadratic_form(x, dt, A, B, C, D=None, init=None):
    """y = M x with M_ts = C_t . (a_t ... a_{s+1}) B_s, built from explicit
    products of the per-step decays (no prefix sums), plus the init and skip
    terms; the final state from the same products."""
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    y = np.zeros((b, L, H, P))
    final = np.zeros((b, H, P, N))
    for bi in range(b):
        for h in range(H):
            g = h // (H // G)
            a = np.exp(dt[bi, :, h] * A[h])
            M = np.zeros((L, L))
            for t in range(L):
                for s in range(t + 1):
                    M[t, s] = np.prod(a[s + 1 : t + 1]) * (C[bi, t, g] @ B[bi, s, g])
            y[bi, :, h, :] = M @ x[bi, :, h, :]
            for s in range(L):
                final[bi, h] += np.prod(a[s + 1 :]) * np.outer(x[bi, s, h], B[bi, s, g])
            if init is not None:
                for t in range(L):
                    y[bi, t, h, :] += np.prod(a[: t + 1]) * (init[bi, h] @ C[bi, t, g])
                final[bi, h] += np.prod(a) * init[bi, h]
            if D is not None:
                y[bi, :, h, :] += D[h] * x[bi, :, h, :]
    return y, final


@pytest.mark.parametrize("G", [1, 2])
@pytest.mark.parametrize("seed", [0, 1])
def test_quadratic_form(G, seed):
    c = rand_case(np.random.default_rng(seed), G=G)
    y, final = oracle.forward(**c)
    yq, fq = quadratic_form(**c)
    assert rel(y, yq) < 1e-12
    assert rel(final, fq) < 1e-12


# ---------------------------------------------------------------- closed forms
def test_linear_attention_exact():
    """a = 1 (A = 0): causal linear attention, exact on small integers."""
    rng = np.random.default_rng(3)
    L, N = 9, 3
    x = rng.integers(-4, 5, (1, L, 1, 1)).astype(float)
    B = rng.integers(-3, 4, (1, L, 1, N)).astype(float)
    C = rng.integers(-3, 4, (1, L, 1, N)).astype(float)
    y, _ = oracle.forward(x, np.full((1, L, 1), 0.37), np.zeros(1), B, C)
    xi, Bi, Ci = (v.astype(int) for v in (x, B, C))
    want = [sum(int(Ci[0, i, 0] @ Bi[0, j, 0]) * int(xi[0, j, 0, 0]) for j in range(i + 1))
            for i in range(L)]
    assert y.ravel().tolist() == [float(v) for v in want]


@pytest.mark.parametrize("gamma", [0.5, 0.9, 0.999])
def test_retnet_constant_decay(gamma):
    """Constant a = gamma, N = P = 1, B = C = x = 1: y_i = (1 - gamma^(i+1)) / (1 - gamma)."""
    L = 50
    one = np.ones((1, L, 1, 1))
    y, _ = oracle.forward(one, np.full((1, L, 1), -math.log(gamma)), np.array([-1.0]), one, one)
    want = [(1 - gamma ** (i + 1)) / (1 - gamma) for i in range(L)]
    np.testing.assert_allclose(y.ravel(), want, rtol=1e-12, atol=0)


def test_memoryless_limit():
    """Very fast decay forgets everything before the current step."""
    c = rand_case(np.random.default_rng(4), with_init=True)
    c["dt"] = np.full_like(c["dt"], 60.0)   # dt * A <= -30, a <= 1e-13
    y, final = oracle.forward(**c)
    G = c["B"].shape[2]
    H = c["x"].shape[2]
    for h in range(H):
        g = h // (H // G)
        cb = np.einsum("bln,bln->bl", c["C"][:, :, g], c["B"][:, :, g])
        want = (cb[..., None] + c["D"][h]) * c["x"][:, :, h, :]
        np.testing.assert_allclose(y[:, :, h, :], want, rtol=0, atol=1e-10)


# ---------------------------------------------------------------- invariants
@pytest.mark.parametrize("Q", [1, 2, 4, 5, 8, 16, 37, 64])
def test_chunk_invariance(Q):
    """The chunked decomposition (every step of it) equals the recurrence."""
    c = rand_case(np.random.default_rng(5), b=2, L=37, H=4, P=3, N=4, G=2)
    y, final, bnd = oracle.forward(**c, chunk=Q)
    yc, fc, inter = chunked.forward_chunked(**c, Q=Q)
    assert rel(yc, y) < 1e-12
    assert rel(fc, final) < 1e-12
    assert rel(inter["hprev"], bnd) < 1e-12


def test_chunk_state_is_state_from_zero():
    """S_c is the state a chunk reaches on its own, started from zero."""
    c = rand_case(np.random.default_rng(6), b=1, L=20, H=2, P=2, N=3)
    Q = 8
    cs = chunked.chunk_cumsum(c["dt"], c["A"], Q)
    S = chunked.chunk_state(c["x"], c["B"], cs, Q)
    for ci in range(3):
        s, e = ci * Q, min(ci * Q + Q, 20)
        _, f = oracle.forward(c["x"][:, s:e], c["dt"][:, s:e], c["A"], c["B"][:, s:e], c["C"][:, s:e])
        assert rel(S[:, ci], f) < 1e-12


def test_chunk_decay_is_product():
    """exp of the last prefix entry is the product of the chunk's decays."""
    rng = np.random.default_rng(7)
    dt = np.exp(rng.uniform(-5, 0, (2, 30, 3)))
    A = -rng.uniform(1, 16, 3)
    cs = chunked.chunk_cumsum(dt, A, 8)
    for c0 in range(4):
        s, e = c0 * 8, min(c0 * 8 + 8, 30)
        want = np.prod(np.exp(dt[:, s:e, :] * A), axis=1)
        np.testing.assert_allclose(np.exp(cs[:, :, c0, e - s - 1]), want, rtol=1e-13)


def test_page5_interchunk_formula_without_weights_is_wrong():
    """The summary page's inter-chunk update omits the within-chunk weights
    exp(cs_e - cs_j); dropping them breaks agreement with the recurrence,
    which is why the oracle keeps them."""
    c = rand_case(np.random.default_rng(8), b=1, L=32, H=2, P=2, N=3, with_init=False)
    Q = 8
    y, _ = oracle.forward(**c)
    cs = chunked.chunk_cumsum(c["dt"], c["A"], Q)
    bad = chunked.chunk_state(c["x"], c["B"], np.zeros_like(cs), Q)   # weights all 1
    hprev, _ = chunked.state_passing(bad, cs, None, L=32, Q=Q)
    yin = chunked.chunk_scan_intra(chunked.chunk_cb(c["C"], c["B"], Q), cs, c["x"], Q)
    ybad = chunked.output_combine(yin, c["C"], cs, hprev, c["x"], c["D"], Q)
    assert rel(ybad, y) > 1e-3


def test_split_call_bitwise():
    """Composition law: forward(0:L) == forward(0:k) then forward(k:L, init=final)."""
    c = rand_case(np.random.default_rng(9), b=2, L=40, H=3, P=4, N=5)
    y, final = oracle.forward(**c)
    k = 17
    sl = lambda v, a, b_: v[:, a:b_]
    y1, f1 = oracle.forward(sl(c["x"], 0, k), sl(c["dt"], 0, k), c["A"], sl(c["B"], 0, k),
                            sl(c["C"], 0, k), c["D"], c["init"])
    y2, f2 = oracle.forward(sl(c["x"], k, 40), sl(c["dt"], k, 40), c["A"], sl(c["B"], k, 40),
                            sl(c["C"], k, 40), c["D"], f1)
    assert np.array_equal(np.concatenate([y1, y2], axis=1), y)
    assert np.array_equal(f2, final)


def test_decode_equals_forward():
    c = rand_case(np.random.default_rng(10), b=2, L=11, H=4, P=3, N=5, G=2)
    y, final = oracle.forward(**c)
    state = c["init"].copy()
    for t in range(11):
        yt, state = oracle.decode_step(state, c["x"][:, t], c["dt"][:, t], c["A"], c["B"][:, t],
                                       c["C"][:, t], c["D"])
        assert np.array_equal(yt, y[:, t])
    assert np.array_equal(state, final)


def test_semiseparable_rank_bound():
    """Every block strictly below the diagonal of M has rank <= N."""
    rng = np.random.default_rng(11)
    L, N = 24, 3
    c = rand_case(rng, b=1, L=L, H=1, P=1, N=N, with_D=False, with_init=False)
    M = np.zeros((L, L))
    for s in range(L):
        e = np.zeros((1, L, 1, 1))
        e[0, s] = 1.0
        M[:, s] = oracle.forward(e, c["dt"], c["A"], c["B"], c["C"])[0].ravel()
    assert np.allclose(np.triu(M, 1), 0)
    for i0 in range(1, L):
        for j0 in range(1, i0 + 1):
            sv = np.linalg.svd(M[i0:, :j0], compute_uv=False)
            assert np.sum(sv > 1e-10 * sv[0]) <= N
    assert np.linalg.matrix_rank(M) == L   # the whole M is not low rank


def test_linearity_and_gauge():
    rng = np.random.default_rng(12)
    c1 = rand_case(rng)
    c2 = rand_case(rng)
    c2.update({k: c1[k] for k in ("dt", "A", "B", "C", "D")})
    al, be = 0.7, -1.3
    mix = dict(c1, x=al * c1["x"] + be * c2["x"], init=al * c1["init"] + be * c2["init"])
    y1, f1 = oracle.forward(**c1)
    y2, f2 = oracle.forward(**c2)
    ym, fm = oracle.forward(**mix)
    assert rel(ym, al * y1 + be * y2) < 1e-12
    assert rel(fm, al * f1 + be * f2) < 1e-12
    s = 3.0
    yg, _ = oracle.forward(**dict(c1, B=c1["B"] * s, C=c1["C"] / s, init=c1["init"] * s))
    assert rel(yg, y1) < 1e-12


def test_mamba1_scan_reduction():
    """Mamba review page, section 3.3: its scan discretises B as dt*B and
    keeps a per-channel diagonal A.  With A constant over the state index and
    one channel per head, it equals this layer run on x pre-multiplied by dt.
    The loop below is our own transcription of that scan."""
    rng = np.random.default_rng(13)
    Bt, L, Dch, N = 2, 15, 3, 4
    x = rng.standard_normal((Bt, L, Dch))
    delta = np.exp(rng.uniform(-4, 0, (Bt, L, Dch)))
    Ad = -rng.uniform(0.5, 3, Dch)
    A = np.repeat(Ad[:, None], N, axis=1)            # (D, N), constant along N
    Bm = rng.standard_normal((Bt, L, N))
    Cm = rng.standard_normal((Bt, L, N))
    ys = np.zeros((Bt, L, Dch))
    h = np.zeros((Bt, Dch, N))
    for t in range(L):
        dA = np.exp(delta[:, t, :, None] * A[None])
        dBx = delta[:, t, :, None] * Bm[:, t, None, :] * x[:, t, :, None]
        h = dA * h + dBx
        ys[:, t] = (h * Cm[:, t, None, :]).sum(-1)
    y, _ = oracle.forward((delta * x)[..., None], delta, Ad, Bm[:, :, None, :], Cm[:, :, None, :])
    assert rel(y[..., 0], ys) < 1e-12


def test_empty_sequence():
    rng = np.random.default_rng(14)
    c = rand_case(rng, L=0)
    y, final = oracle.forward(**c)
    assert y.shape == (2, 0, 4, 3)
    assert np.array_equal(final, c["init"])
    yc, fc, _ = chunked.forward_chunked(**c, Q=4)
    assert np.array_equal(fc, c["init"])
