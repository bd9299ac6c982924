"""Pins of oracle.gated_rmsnorm (the normalisation after the gate).

  * silu against its identities: silu(0) = 0, silu(z) - silu(-z) = z, and its
    limits (silu(z) -> z for large z, -> 0 for very negative z);
  * with unit weight each group of the output has mean square
    ms / (ms + eps) exactly, ms the group's mean square of y * silu(z);
  * scale invariance in y when eps = 0, and per-group independence;
  * the weight multiplies channel by channel.
"""
import numpy as np
import pytest

import oracle


def test_silu_identities_and_limits():
    z = np.array([[-50.0, -3.0, -0.5, 0.0, 0.5, 3.0, 50.0]])[None]     # [1, 1, 7] as [.., H=1, P=7]
    y = np.ones_like(z)
    w = np.ones(7)
    g = lambda zz: oracle.gated_rmsnorm(y, zz, w, eps=1e300) * np.sqrt(1e300)   # eps dominates: out ~ g
    s1, s2 = g(z), g(-z)
    assert abs(s1[0, 0, 3]) < 1e-300
    assert np.allclose(s1 - s2, z, rtol=1e-9, atol=1e-12)
    assert abs(s1[0, 0, -1] - 50.0) < 1e-9 and abs(s1[0, 0, 0]) < 1e-19


@pytest.mark.parametrize("groups", [1, 2, 8])
def test_unit_weight_mean_square(groups):
    rng = np.random.default_rng(1)
    y = rng.standard_normal((3, 5, 4, 16))
    z = rng.standard_normal((3, 5, 4, 16))
    eps = 0.25
    out = oracle.gated_rmsnorm(y, z, np.ones(64), norm_groups=groups, eps=eps)
    g = (y * z / (1 + np.exp(-z))).reshape(15, groups, 64 // groups)
    ms = (g * g).mean(-1)
    got = (out.reshape(15, groups, 64 // groups) ** 2).mean(-1)
    assert np.allclose(got, ms / (ms + eps), rtol=1e-13)


def test_scale_invariance_and_group_independence():
    rng = np.random.default_rng(2)
    y = rng.standard_normal((2, 7, 2, 32))
    z = rng.standard_normal((2, 7, 2, 32))
    w = rng.standard_normal(64)
    a = oracle.gated_rmsnorm(y, z, w, norm_groups=2, eps=0.0)
    b = oracle.gated_rmsnorm(3.7 * y, z, w, norm_groups=2, eps=0.0)
    assert np.allclose(a, b, rtol=1e-13)
    y2 = y.copy()
    y2[..., 1, :] *= 5.0                          # changes only the second group's scale
    c = oracle.gated_rmsnorm(y2, z, w, norm_groups=2, eps=0.0)
    assert np.allclose(c, a, rtol=1e-13)


def test_weight_is_per_channel():
    rng = np.random.default_rng(3)
    y = rng.standard_normal((4, 3, 8))
    z = rng.standard_normal((4, 3, 8))
    w = rng.standard_normal(24)
    a = oracle.gated_rmsnorm(y, z, w, eps=1e-5)
    b = oracle.gated_rmsnorm(y, z, np.ones(24), eps=1e-5)
    assert np.allclose(a, b * w.reshape(3, 8), rtol=1e-14)
