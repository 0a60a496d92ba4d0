"""Pins of the oracle's RoPE (pairs (m, m + d/2), theta_m = base**(-2m/d)).

Checked against explicit rotation matrices built in pure Python, and against
the group properties the correction rotation relies on (Jet-Long technical
summary, Methodology item 2: rotations compose additively)."""

import math

import numpy as np
import pytest

from oracle import rope, rope_theta
from oracle.brute import matvec, rotation_matrix


def test_theta_closed_form():
    th = rope_theta(8, 10000.0)
    assert th[0] == 1.0
    np.testing.assert_allclose(th, [1.0, 0.1, 0.01, 0.001], rtol=1e-15)
    th = rope_theta(128, 1e6)
    np.testing.assert_allclose(th[1], 1e6 ** (-1 / 64), rtol=1e-15)
    assert np.all(np.diff(th) < 0)


@pytest.mark.parametrize("d,base", [(2, 10000.0), (4, 10.0), (8, 10000.0), (16, 1e6)])
def test_against_rotation_matrix(d, base):
    rng = np.random.default_rng(d)
    x = rng.standard_normal((7, d))
    pos = np.array([0, 1, 5, 17, 1000, -3, 131071])
    got = rope(x, pos, rope_theta(d, base))
    for n in range(7):
        want = matvec(rotation_matrix(d, int(pos[n]), base), list(x[n]))
        np.testing.assert_allclose(got[n], want, rtol=0, atol=1e-12)


def test_d2_is_complex_rotation():
    # d = 2, theta_0 = 1: (1, 0) at position p is (cos p, sin p)
    p = np.array([0, 1, 2, 3, 100, 12345])
    got = rope(np.tile([[1.0, 0.0]], (6, 1)), p, rope_theta(2, 10000.0))
    np.testing.assert_allclose(got[:, 0], np.cos(p), atol=1e-15)
    np.testing.assert_allclose(got[:, 1], np.sin(p), atol=1e-15)


def test_group_properties():
    rng = np.random.default_rng(0)
    d = 128
    th = rope_theta(d, 1e6)
    x = rng.standard_normal((64, 3, d))
    a = rng.integers(-50000, 131072, 64)
    b = rng.integers(-50000, 131072, 64)
    # R(0) = I
    assert np.array_equal(rope(x, np.zeros(64, np.int64), th), x)
    # norm preserved per head vector
    np.testing.assert_allclose(np.linalg.norm(rope(x, a, th), axis=-1), np.linalg.norm(x, axis=-1),
                               rtol=1e-13)
    # additive composition R(a) R(b) = R(a + b)
    np.testing.assert_allclose(rope(rope(x, b, th), a, th), rope(x, a + b, th), atol=5e-10)
    # inverse
    np.testing.assert_allclose(rope(rope(x, a, th), -a, th), x, atol=5e-10)
    # relative property: <R(a)u, R(b)w> depends on b - a only
    u = x[:, 0]
    w = x[:, 1]
    lhs = np.sum(rope(u[:, None], a, th) * rope(w[:, None], b, th), axis=-1)
    rhs = np.sum(u[:, None] * rope(w[:, None], b - a, th), axis=-1)
    np.testing.assert_allclose(lhs, rhs, atol=1e-9)
