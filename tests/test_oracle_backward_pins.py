"""Pins of the backward oracle (oracle.backward), none of which compares the
oracle with itself.

The loss is sum(dy * y) + sum(dfinal * final_state).  Its gradient is fixed
by:
  * central finite differences of the forward oracle (an independent code
    path: the forward recurrence, differenced numerically), along random
    directions for every input and element by element on a few entries;
  * PyTorch float64 autograd of the explicit quadratic form
    Y = (L o C B^T) X + exp(cs) C init^T + D X with L_ij = prod a (Mamba-2
    review, docsaid.org, section "SSM を一つの行列として書く"): a different
    formula differentiated by a different machine;
  * exact special cases: dD = sum dy . x, and with dy = 0 every gradient is
    that of sum(dfinal * final) alone.
test_oracle_backward_mutations.py checks that plausible mistakes in the
oracle fail these pins.
"""
import numpy as np
import pytest
import torch

import oracle


def rel(a, r):
    a, r = np.asarray(a, np.float64), np.asarray(r, np.float64)
    return float(np.linalg.norm(a - r) / max(np.linalg.norm(r), 1e-30))


def case(rng, b=2, L=19, H=4, P=3, N=5, G=2, with_D=True, with_init=True, with_final=True):
    c = dict(
        x=rng.standard_normal((b, L, H, P)),
        dt=np.exp(rng.uniform(np.log(1e-2), np.log(0.5), (b, L, H))),
        A=-rng.uniform(0.5, 3.0, H),
        B=rng.standard_normal((b, L, G, N)) / np.sqrt(N),
        C=rng.standard_normal((b, L, G, N)) / np.sqrt(N),
        D=rng.standard_normal(H) if with_D else None,
        init=rng.standard_normal((b, H, P, N)) if with_init else None,
    )
    dy = rng.standard_normal((b, L, H, P))
    df = rng.standard_normal((b, H, P, N)) if with_final else None
    return c, dy, df


def loss(c, dy, df):
    y, fin = oracle.forward(**c)
    out = float(np.sum(dy * y))
    if df is not None:
        out += float(np.sum(df * fin))
    return out


GRAD_OF = {"x": "dx", "dt": "ddt", "A": "dA", "B": "dB", "C": "dC", "D": "dD", "init": "dinit"}


@pytest.mark.parametrize("seed", [0, 1])
@pytest.mark.parametrize("name", sorted(GRAD_OF))
def test_directional_finite_difference(seed, name):
    rng = np.random.default_rng(seed)
    c, dy, df = case(rng)
    gr = oracle.backward(c["x"], c["dt"], c["A"], c["B"], c["C"], c["D"], c["init"], dy, df)
    v = rng.standard_normal(c[name].shape)
    eps = 1e-6
    cp, cm = dict(c), dict(c)
    cp[name] = c[name] + eps * v
    cm[name] = c[name] - eps * v
    fd = (loss(cp, dy, df) - loss(cm, dy, df)) / (2 * eps)
    an = float(np.sum(gr[GRAD_OF[name]] * v))
    assert abs(fd - an) <= 1e-7 * max(1.0, abs(fd)), (name, fd, an)


def test_elementwise_finite_difference():
    rng = np.random.default_rng(3)
    c, dy, df = case(rng, b=1, L=9, H=2, P=2, N=3, G=1)
    gr = oracle.backward(c["x"], c["dt"], c["A"], c["B"], c["C"], c["D"], c["init"], dy, df)
    eps = 1e-6
    for name in sorted(GRAD_OF):
        flat = c[name].reshape(-1)
        for idx in rng.choice(flat.size, size=min(4, flat.size), replace=False):
            e = np.zeros_like(flat)
            e[idx] = eps
            cp, cm = dict(c), dict(c)
            cp[name] = (flat + e).reshape(c[name].shape)
            cm[name] = (flat - e).reshape(c[name].shape)
            fd = (loss(cp, dy, df) - loss(cm, dy, df)) / (2 * eps)
            an = gr[GRAD_OF[name]].reshape(-1)[idx]
            assert abs(fd - an) <= 1e-7 * max(1.0, abs(fd)), (name, idx, fd, an)


def quadratic_form_torch(x, dt, A, B, C, D, init):
    """y and final state of the forward map written as the masked
    (attention-like) matrix form, in torch float64 (differentiable)."""
    b, L, H, P = x.shape
    G = B.shape[2]
    ys, fins = [], []
    for bi in range(b):
        yh, fh = [], []
        for h in range(H):
            g = h // (H // G)
            cs = torch.cumsum(dt[bi, :, h] * A[h], 0)                        # cs_i = sum_{k<=i} dA_k
            diff = cs[:, None] - cs[None, :]
            Lm = torch.where(torch.tril(torch.ones(L, L, dtype=torch.bool)), torch.exp(torch.tril(diff)),
                             torch.zeros((), dtype=torch.float64))
            M = Lm * (C[bi, :, g] @ B[bi, :, g].T)                            # (L o C B^T)
            y = M @ x[bi, :, h]
            fin = (torch.exp(cs[-1] - cs)[:, None] * x[bi, :, h]).T @ B[bi, :, g]
            if init is not None:
                y = y + torch.exp(cs)[:, None] * (C[bi, :, g] @ init[bi, h].T)
                fin = fin + torch.exp(cs[-1]) * init[bi, h]
            if D is not None:
                y = y + D[h] * x[bi, :, h]
            yh.append(y)
            fh.append(fin)
        ys.append(torch.stack(yh, 1))
        fins.append(torch.stack(fh, 0))
    return torch.stack(ys, 0), torch.stack(fins, 0)


@pytest.mark.parametrize("G", [1, 2])
@pytest.mark.parametrize("with_D,with_init,with_final", [(True, True, True), (False, False, False),
                                                         (True, False, True)])
def test_autograd_of_quadratic_form(G, with_D, with_init, with_final):
    rng = np.random.default_rng(10 + G)
    c, dy, df = case(rng, G=G, with_D=with_D, with_init=with_init, with_final=with_final)
    t = {k: (None if v is None else torch.tensor(v, dtype=torch.float64, requires_grad=True)) for k, v in c.items()}
    y, fin = quadratic_form_torch(**t)
    ls = (y * torch.tensor(dy)).sum()
    if df is not None:
        ls = ls + (fin * torch.tensor(df)).sum()
    ls.backward()
    gr = oracle.backward(c["x"], c["dt"], c["A"], c["B"], c["C"], c["D"], c["init"], dy, df)
    for name, gname in GRAD_OF.items():
        if t[name] is None:
            continue
        assert rel(gr[gname], t[name].grad.numpy()) < 1e-10, name
    if t["init"] is None:
        # dinit of an absent (zero) init: the autograd of the form with a zero init tensor
        t0 = dict(t)
        t0["init"] = torch.zeros(c["x"].shape[0], c["x"].shape[2], c["x"].shape[3], c["B"].shape[3],
                                 dtype=torch.float64, requires_grad=True)
        y, fin = quadratic_form_torch(**t0)
        ls = (y * torch.tensor(dy)).sum() + (0 if df is None else (fin * torch.tensor(df)).sum())
        ls.backward()
        assert rel(gr["dinit"], t0["init"].grad.numpy()) < 1e-10


def test_skip_gradient_exact():
    rng = np.random.default_rng(5)
    c, dy, df = case(rng)
    gr = oracle.backward(c["x"], c["dt"], c["A"], c["B"], c["C"], c["D"], c["init"], dy, df)
    assert np.allclose(gr["dD"], np.einsum("blhp,blhp->h", dy, c["x"]), rtol=1e-13, atol=1e-13)


def test_final_state_only():
    """With dy = 0 only final_state feeds the loss: dx_t = dfinal_weighted B_t with
    the decay from t to the end, dC = 0, dinit = prod(a) dfinal."""
    rng = np.random.default_rng(6)
    c, dy, df = case(rng, b=1, H=2, G=1)
    dy = np.zeros_like(dy)
    gr = oracle.backward(c["x"], c["dt"], c["A"], c["B"], c["C"], c["D"], c["init"], dy, df)
    assert np.abs(gr["dC"]).max() == 0.0 and np.abs(gr["dD"]).max() == 0.0
    cs = np.cumsum(c["dt"][0] * c["A"][None, :], axis=0)                   # [L, H]
    for h in range(2):
        w = np.exp(cs[-1, h] - cs[:, h])                                   # decay from t to the end
        dx = w[:, None] * (df[0, h] @ c["B"][0, :, 0].T).T                  # [L, P]
        assert rel(gr["dx"][0, :, h], dx) < 1e-12
        assert rel(gr["dinit"][0, h], np.exp(cs[-1, h]) * df[0, h]) < 1e-12


def test_linear_in_output_gradients():
    rng = np.random.default_rng(7)
    c, dy, df = case(rng)
    dy2 = rng.standard_normal(dy.shape)
    df2 = rng.standard_normal(df.shape)
    args = (c["x"], c["dt"], c["A"], c["B"], c["C"], c["D"], c["init"])
    g1 = oracle.backward(*args, dy, df)
    g2 = oracle.backward(*args, dy2, df2)
    g3 = oracle.backward(*args, 2 * dy - 3 * dy2, 2 * df - 3 * df2)
    for k in g1:
        assert rel(g3[k], 2 * g1[k] - 3 * g2[k]) < 1e-12, k


def test_long_sequence_crosses_checkpoints():
    """L spans several 64-step checkpoint segments; directional FD still holds."""
    rng = np.random.default_rng(8)
    c, dy, df = case(rng, b=1, L=150, H=2, P=2, N=3, G=1)
    gr = oracle.backward(c["x"], c["dt"], c["A"], c["B"], c["C"], c["D"], c["init"], dy, df)
    for name in ("x", "dt", "A", "init"):
        v = rng.standard_normal(c[name].shape)
        eps = 1e-6
        cp, cm = dict(c), dict(c)
        cp[name] = c[name] + eps * v
        cm[name] = c[name] - eps * v
        fd = (loss(cp, dy, df) - loss(cm, dy, df)) / (2 * eps)
        an = float(np.sum(gr[GRAD_OF[name]] * v))
        assert abs(fd - an) <= 1e-7 * max(1.0, abs(fd)), (name, fd, an)
