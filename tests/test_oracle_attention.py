"""Pins of the oracle's bifocal prefill (distance-routed causal attention,
Jet-Long technical summary, Methodology items 1 and 2).

Each pin is independent of the oracle's own code: a pure-Python brute force,
closed forms, a library causal attention for the cases that reduce to it, and
a separately written three-pass inclusion-exclusion implementation."""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import brute
from oracle.three_pass import prefill_three_pass


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


@pytest.mark.parametrize("L,d,w0,w_pt,base", [
    (1, 2, 1, 4, 10000.0),
    (9, 2, 2, 4, 10000.0),
    (13, 4, 3, 4, 10.0),      # G = 4
    (24, 8, 5, 7, 10000.0),   # G = 4, ragged group
    (17, 4, 0, 5, 10.0),      # w0 = 0: everything remote
    (16, 4, 40, 5, 10.0),     # w0 >= L: everything local
    (30, 8, 6, 30, 100.0),    # G = 1
])
def test_against_pure_python_brute(L, d, w0, w_pt, base):
    q, k, v = _rand((L, 1, d), 1), _rand((L, 1, d), 2), _rand((L, 1, d), 3)
    o, lse = oracle.prefill(q, k, v, w0=w0, w_pretrained=w_pt, rope_base=base)
    ob, lb = brute.prefill_brute(q[:, 0].tolist(), k[:, 0].tolist(), v[:, 0].tolist(), w0, w_pt, base)
    np.testing.assert_allclose(o[:, 0], ob, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse[0], lb, rtol=0, atol=1e-12)


def test_d2_hand_example():
    """d = 2, raw q = k = (1, 0): a score is scale * cos(position difference),
    with the base difference i - j for local pairs and f(i) - f(j) remote.
    L = 4, w_pretrained = 2 (G = 2), w0 = 1 (only the diagonal is local)."""
    L = 4
    q = np.tile([[[1.0, 0.0]]], (L, 1, 1))
    v = np.array([[[1.0, 0.0]], [[0.0, 1.0]], [[2.0, 0.0]], [[0.0, 3.0]]])
    o, lse = oracle.prefill(q, q, v, w0=1, w_pretrained=2, rope_base=10000.0)
    s = 1 / math.sqrt(2)
    c1 = s * math.cos(1.0)
    # row 0: {0}; row 1: f-diff 0, local; row 2: f-diff 1, 1, local;
    # row 3: f-diff 1, 1, 0, local
    want_lse = [s, s + math.log(2), math.log(2 * math.exp(c1) + math.exp(s)),
                math.log(2 * math.exp(c1) + 2 * math.exp(s))]
    np.testing.assert_allclose(lse[0], want_lse, atol=1e-14)
    w3 = np.array([math.exp(c1), math.exp(c1), math.exp(s), math.exp(s)])
    want_o3 = (w3[:, None] * v[:, 0]).sum(0) / w3.sum()
    np.testing.assert_allclose(o[3, 0], want_o3, atol=1e-14)
    np.testing.assert_allclose(o[1, 0], (v[0, 0] + v[1, 0]) / 2, atol=1e-15)


@pytest.mark.parametrize("G_case", [(64, 16, 64), (200, 30, 64), (200, 0, 50)])
def test_zero_query_gives_prefix_mean(G_case):
    L, w0, w_pt = G_case
    q = np.zeros((L, 2, 8))
    k, v = _rand((L, 1, 8), 4), _rand((L, 1, 8), 5)
    o, lse = oracle.prefill(q, k, v, w0=w0, w_pretrained=w_pt, rope_base=10000.0)
    want = np.cumsum(v[:, 0], axis=0) / np.arange(1, L + 1)[:, None]
    for h in range(2):
        np.testing.assert_allclose(o[:, h], want, atol=1e-13)
        np.testing.assert_allclose(lse[h], np.log(np.arange(1, L + 1)), atol=1e-13)


def test_constant_values_pass_through():
    L = 100
    q, k = _rand((L, 2, 16), 6, 3.0), _rand((L, 1, 16), 7, 3.0)
    v = np.broadcast_to(np.linspace(-2, 2, 16), (L, 1, 16)).copy()
    o, _ = oracle.prefill(q, k, v, w0=10, w_pretrained=30, rope_base=10000.0)
    np.testing.assert_allclose(o, np.broadcast_to(v[:, :1], o.shape), atol=1e-12)


def _sdpa_causal(qr, kr, v, scale):
    """Library causal attention in float64 on the CPU; GQA by repeating kv."""
    Hq, Hkv = qr.shape[1], kr.shape[1]
    rep = Hq // Hkv
    Q = torch.from_numpy(qr).permute(1, 0, 2)
    K = torch.from_numpy(kr).permute(1, 0, 2).repeat_interleave(rep, 0)
    V = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(rep, 0)
    o = torch.nn.functional.scaled_dot_product_attention(Q, K, V, is_causal=True, scale=scale)
    s = (Q @ K.transpose(1, 2)) * scale
    s = s.masked_fill(torch.triu(torch.ones(s.shape[-2:], dtype=torch.bool), 1), float("-inf"))
    lse = torch.logsumexp(s, dim=-1)
    return o.permute(1, 0, 2).numpy(), lse.numpy()


@pytest.mark.parametrize("L,w0,w_pt", [(96, 16, 96), (96, 16, 500), (80, 80, 20), (80, 500, 10)])
def test_base_model_recovered(L, w0, w_pt):
    """G = 1 (L <= w_pretrained) or w0 >= L: plain causal RoPE attention at
    absolute positions (English abstract: the base model is recovered exactly
    on short inputs)."""
    d = 16
    q, k, v = _rand((L, 4, d), 8), _rand((L, 2, d), 9), _rand((L, 2, d), 10)
    o, lse = oracle.prefill(q, k, v, w0=w0, w_pretrained=w_pt, rope_base=10000.0)
    th = oracle.rope_theta(d, 10000.0)
    p = np.arange(L)
    o_ref, lse_ref = _sdpa_causal(oracle.rope(q, p, th), oracle.rope(k, p, th), v, 1 / math.sqrt(d))
    np.testing.assert_allclose(o, o_ref, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, atol=1e-12)


def test_w0_zero_is_causal_at_aliased_positions():
    L, d, w_pt = 90, 16, 25            # G = 4
    q, k, v = _rand((L, 4, d), 11), _rand((L, 2, d), 12), _rand((L, 2, d), 13)
    o, lse = oracle.prefill(q, k, v, w0=0, w_pretrained=w_pt, rope_base=10000.0)
    th = oracle.rope_theta(d, 10000.0)
    f = np.arange(L) // 4
    o_ref, lse_ref = _sdpa_causal(oracle.rope(q, f, th), oracle.rope(k, f, th), v, 1 / math.sqrt(d))
    np.testing.assert_allclose(o, o_ref, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, atol=1e-12)


def test_rows_below_window_are_plain_causal_rows():
    L, d, w0, w_pt = 120, 16, 40, 30   # G = 4
    q, k, v = _rand((L, 2, d), 14), _rand((L, 1, d), 15), _rand((L, 1, d), 16)
    o, lse = oracle.prefill(q, k, v, w0=w0, w_pretrained=w_pt, rope_base=10000.0)
    th = oracle.rope_theta(d, 10000.0)
    p = np.arange(L)
    o_ref, lse_ref = _sdpa_causal(oracle.rope(q, p, th), oracle.rope(k, p, th), v, 1 / math.sqrt(d))
    np.testing.assert_allclose(o[:w0], o_ref[:w0], atol=1e-12)
    np.testing.assert_allclose(lse[:, :w0], lse_ref[:, :w0], atol=1e-12)
    # and later rows do differ (the remote grid is in use)
    assert np.abs(o[w0:] - o_ref[w0:]).max() > 1e-3


def test_sampled_rows_match_full():
    L, d = 300, 32
    q, k, v = _rand((L, 4, d), 17), _rand((L, 2, d), 18), _rand((L, 2, d), 19)
    kw = dict(w0=20, w_pretrained=80, rope_base=10000.0)
    o, lse = oracle.prefill(q, k, v, **kw)
    rows = np.array([0, 1, 19, 20, 21, 150, 299])
    os_, ls_ = oracle.prefill(q, k, v, rows=rows, **kw)
    np.testing.assert_allclose(os_, o[rows], atol=1e-14)
    np.testing.assert_allclose(ls_, lse[:, rows], atol=1e-14)


@pytest.mark.parametrize("L,d,w0,w_pt,Hq,Hkv", [(256, 64, 16, 64, 1, 1), (200, 32, 33, 50, 4, 2),
                                                 (150, 16, 0, 40, 2, 1), (64, 16, 100, 20, 2, 2)])
def test_three_pass_merge_is_exact(L, d, w0, w_pt, Hq, Hkv):
    """The inclusion-exclusion merge of three passes reproduces the routed
    output (Methodology item 2), up to fp64 rounding."""
    q, k, v = _rand((L, Hq, d), 20), _rand((L, Hkv, d), 21), _rand((L, Hkv, d), 22)
    kw = dict(w0=w0, w_pretrained=w_pt, rope_base=10000.0)
    o, lse = oracle.prefill(q, k, v, **kw)
    o3, lse3 = prefill_three_pass(q, k, v, **kw)
    np.testing.assert_allclose(o3, o, atol=1e-13)
    np.testing.assert_allclose(lse3, lse, atol=1e-13)


def test_varlen_sequences_are_independent():
    d = 16
    lens = [37, 1, 90]
    cu = np.cumsum([0] + lens)
    q, k, v = _rand((cu[-1], 2, d), 23), _rand((cu[-1], 1, d), 24), _rand((cu[-1], 1, d), 25)
    kw = dict(w0=9, w_pretrained=30, rope_base=10000.0)
    outs = oracle.prefill_varlen(q, k, v, cu, **kw)
    for b in range(3):
        o, lse = oracle.prefill(q[cu[b]:cu[b + 1]], k[cu[b]:cu[b + 1]], v[cu[b]:cu[b + 1]], **kw)
        assert np.array_equal(outs[b][0], o) and np.array_equal(outs[b][1], lse)


def test_explicit_head_map():
    L, d = 50, 8
    q, k, v = _rand((L, 3, d), 26), _rand((L, 2, d), 27), _rand((L, 2, d), 28)
    kw = dict(w0=5, w_pretrained=20, rope_base=10000.0)
    o, _ = oracle.prefill(q, k, v, q_to_kv=[1, 0, 1], **kw)
    o1, _ = oracle.prefill(q[:, :1], k[:, 1:2], v[:, 1:2], **kw)
    np.testing.assert_allclose(o[:, 0], o1[:, 0], atol=0)
