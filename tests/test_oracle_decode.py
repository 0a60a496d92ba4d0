"""Pins of the oracle's decode step with the correction rotation Delta
(Jet-Long technical summary, Methodology item 2: the cache keeps base keys at
absolute positions; the query and cached keys are rotated on the fly)."""

import math

import numpy as np
import pytest

import oracle
from oracle import brute


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("L,d,w0,w_pt", [(1, 4, 2, 3), (11, 4, 3, 3), (20, 8, 4, 6), (20, 8, 0, 6),
                                          (20, 8, 30, 6), (15, 2, 2, 20)])
def test_against_brute(L, d, w0, w_pt):
    base = 100.0
    th = oracle.rope_theta(d, base)
    k_raw, v = _rand((L, 1, d), 1), _rand((L, 1, d), 2)
    K = oracle.rope(k_raw, np.arange(L), th)             # cache: base keys at absolute j
    qb = oracle.rope(_rand((1, 1, d), 3), np.array([L - 1]), th)[:, 0]
    o, lse = oracle.decode(qb, K, v, L, w0=w0, w_pretrained=w_pt, rope_base=base)
    ob, lb = brute.decode_brute(qb[0].tolist(), K[:, 0].tolist(), v[:, 0].tolist(), L, w0, w_pt, base)
    np.testing.assert_allclose(o[0], ob, atol=1e-12)
    np.testing.assert_allclose(lse[0], lb, atol=1e-12)


@pytest.mark.parametrize("L,w0,w_pt", [(64, 8, 16), (64, 8, 64), (65, 8, 64), (129, 8, 64),
                                        (200, 50, 33), (100, 0, 30)])
def test_equals_last_prefill_row(L, w0, w_pt):
    """Decode at length L equals the last row of bifocal prefill at length L
    when the cache holds the prefill's keys rotated at absolute positions."""
    d, Hq, Hkv = 32, 4, 2
    base = 10000.0
    th = oracle.rope_theta(d, base)
    q, k, v = _rand((L, Hq, d), 4), _rand((L, Hkv, d), 5), _rand((L, Hkv, d), 6)
    o_p, lse_p = oracle.prefill(q, k, v, w0=w0, w_pretrained=w_pt, rope_base=base, rows=[L - 1])
    K = oracle.rope(k, np.arange(L), th)
    qb = oracle.rope(q[L - 1:L], np.array([L - 1]), th)[0]
    o, lse = oracle.decode(qb, K, v, L, w0=w0, w_pretrained=w_pt, rope_base=base)
    np.testing.assert_allclose(o, o_p[0], atol=1e-12)
    np.testing.assert_allclose(lse, lse_p[:, 0], atol=1e-12)


def test_boundary_crossing_changes_only_g():
    """Across L = w_pt -> w_pt + 1 the cache is the same array, G steps from 1
    to 2, and the step at L = w_pt is plain causal attention."""
    d, w_pt, w0 = 16, 64, 8
    th = oracle.rope_theta(d, 1e4)
    L1 = w_pt + 1
    K = oracle.rope(_rand((L1, 1, d), 7), np.arange(L1), th)
    V = _rand((L1, 1, d), 8)
    K_before = K.copy()
    q = _rand((1, d), 9)
    assert oracle.group_size(w_pt, w_pt) == 1 and oracle.group_size(w_pt + 1, w_pt) == 2
    o, lse = oracle.decode(q, K, V, w_pt, w0=w0, w_pretrained=w_pt, rope_base=1e4)
    s = (K[:w_pt, 0] @ q[0]) / math.sqrt(d)
    m = s.max()
    e = np.exp(s - m)
    np.testing.assert_allclose(o[0], e @ V[:w_pt, 0] / e.sum(), atol=1e-13)
    np.testing.assert_allclose(lse[0], m + math.log(e.sum()), atol=1e-13)
    oracle.decode(q, K, V, L1, w0=w0, w_pretrained=w_pt, rope_base=1e4)
    assert np.array_equal(K, K_before)


def test_zero_length_is_empty():
    o, lse = oracle.decode(np.ones((2, 4)), np.ones((3, 1, 4)), np.ones((3, 1, 4)), 0,
                           w0=1, w_pretrained=2, rope_base=10.0)
    assert o.shape == (2, 4) and lse.shape == (2,)
