"""Separately written fp64 three-pass inclusion-exclusion attention.

TEST INFRASTRUCTURE ONLY (see ``oracle/jetlong.py``).  Used to pin the pages'
claim that the three-pass merge reproduces the distance-routed output exactly
(Jet-Long technical summary, Methodology item 2, "Inference efficiency
mechanisms": inclusion-exclusion merge of three FlashAttention passes,
stabilised with LogSumExp statistics, without a boolean mask matrix).

The three passes are plain dense softmax passes, each with its own
(output, LSE) pair:
  pass 1  local window (0 <= i - j < w0), base-rotated q and k
  pass 2  full causal (j <= i), aliased-position q and k
  pass 3  local window, aliased-position q and k
and the merge is  out = (z1 o1 + z2 o2 - z3 o3) / (z1 + z2 - z3),
z_k = exp(lse_k - M), M = max(lse_1, lse_2), lse = M + log(z1 + z2 - z3).

The windowed passes are dense passes whose out-of-window scores are -inf,
which is how a standard attention routine with a sliding window restricts its
keys.  Small inputs only.
"""

from __future__ import annotations

import math

import numpy as np

from .jetlong import group_size, remote_pos, rope, rope_theta


def _pass(qh, kh, vh, allowed, scale):
    s = scale * (qh @ kh.T)
    s = np.where(allowed, s, -np.inf)
    with np.errstate(invalid="ignore", divide="ignore"):
        m = s.max(axis=1)
        e = np.exp(s - m[:, None])
        z = e.sum(axis=1)
        return (e @ vh) / z[:, None], m + np.log(z)


def prefill_three_pass(q, k, v, *, w0, w_pretrained, rope_base, scale=None):
    """q: [L, Hq, d], k, v: [L, Hkv, d]; GQA by h // (Hq / Hkv).
    Returns (o [L, Hq, d], lse [Hq, L])."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    L, Hq, d = q.shape
    Hkv = k.shape[1]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    G = group_size(L, w_pretrained)
    th = rope_theta(d, rope_base)
    p = np.arange(L)
    f = remote_pos(p, G)
    qb, kb = rope(q, p, th), rope(k, p, th)
    qr, kr = rope(q, f, th), rope(k, f, th)
    i = p[:, None]
    j = p[None, :]
    causal = j <= i
    window = causal & (i - j < w0)
    o = np.zeros_like(q)
    lse = np.zeros((Hq, L))
    for h in range(Hq):
        g = h // (Hq // Hkv)
        o1, l1 = _pass(qb[:, h], kb[:, g], v[:, g], window, scale)
        o2, l2 = _pass(qr[:, h], kr[:, g], v[:, g], causal, scale)
        o3, l3 = _pass(qr[:, h], kr[:, g], v[:, g], window, scale)
        # rows with an empty window (w0 == 0) carry lse = -inf and weight 0
        l1 = np.where(np.isfinite(l1), l1, -np.inf)
        l3 = np.where(np.isfinite(l3), l3, -np.inf)
        o1 = np.nan_to_num(o1)
        o3 = np.nan_to_num(o3)
        M = np.maximum(l1, l2)
        z1 = np.exp(l1 - M)
        z2 = np.exp(l2 - M)
        z3 = np.exp(l3 - M)
        Z = z1 + z2 - z3
        o[:, h] = (z1[:, None] * o1 + z2[:, None] * o2 - z3[:, None] * o3) / Z[:, None]
        lse[h] = M + np.log(Z)
    return o, lse
