"""fp64 CPU oracle of Jet-Long dynamic bifocal RoPE attention.

TEST INFRASTRUCTURE ONLY.  Only tests, the smoke check and the benchmark's CPU
baseline leg may import this module.  The HIP library never calls it, and it
shares no code, table or constant with the HIP path.

Sources (the pages about "Jet-Long: Efficient Long-Context Extension with
Dynamic Bifocal RoPE"):
  [TS-M1]  technical summary (gist.science; Spanish "Resumen Técnico: Jet-Long",
           with German and Japanese translations), Methodology item 1,
           "Dynamic Bifocal RoPE": local window w0 with classical RoPE, remote
           map f, group-size equation G.
  [TS-M2]  same summary, Methodology item 2, "Inference efficiency
           mechanisms": the on-the-fly correction rotation Delta for
           generation, and the three-pass inclusion-exclusion attention merge
           stabilised with LogSumExp statistics.
  [ABS]    the authors' English abstract (chatpaper.ai page): exact recovery of
           the base model on short inputs.

What is computed here is the plain definition of the result: causal softmax
attention in which every (query i, key j) score is taken from base RoPE at the
absolute positions when the pair is closer than w0, and from RoPE at the
aliased positions f(i), f(j) otherwise [TS-M1].  The three-pass merge of
[TS-M2] is a faster route to the same numbers; a separately written three-pass
version lives in ``oracle/three_pass.py`` and is only used to pin that claim.

Readings where the pages are silent (each is listed with its reason in the
design notes):
  R1  local iff 0 <= i - j < w0 (w0 keys including the query's own); remote
      iff i - j >= w0.  Locality is by relative distance.
  R3  prefill uses one G per sequence, from that sequence's full length L.
  R4  decode: L counts the cached keys including the current token; the query
      sits at position L - 1.
  R5  no extra remote-position offset: f is applied to query and key alike.
  R6  the query is aliased too: remote scores use R(f(i)) q and R(f(j)) k.
  R7  RoPE pairs dimension m with m + d/2 and uses theta_m = base**(-2m/d)
      (the rotary layout of the Qwen3 models the pages evaluate).
  R9  softmax scale 1/sqrt(d) unless given.
  R10 GQA: kv head of q head h is h // (Hq / Hkv) unless a map is given.
  R11 LSE is the natural log of sum_j exp(scale * q.k), per (head, row).
  R12 decode receives q already rotated by base RoPE at position L - 1.
  R14 L = 0 is empty; w0 = 0 routes every pair to the remote grid.
"""

from __future__ import annotations

from typing import Optional, Sequence

import numpy as np


# --------------------------------------------------------------------------
# position mapper [TS-M1]
# --------------------------------------------------------------------------

def group_size(L: int, w_pretrained: int) -> int:
    """G = max(1, ceil(L / w_pretrained)) with exact Python integers [TS-M1]."""
    L = int(L)
    w_pretrained = int(w_pretrained)
    if w_pretrained <= 0 or L < 0:
        raise ValueError("group_size needs L >= 0 and w_pretrained >= 1")
    ceil_div = -((-L) // w_pretrained)
    return max(1, ceil_div)


def remote_pos(x, G: int):
    """f(x) = floor(x / G) for non-negative integer positions [TS-M1]."""
    if G < 1:
        raise ValueError("G must be >= 1")
    return np.asarray(x, dtype=np.int64) // np.int64(G)


# --------------------------------------------------------------------------
# RoPE (R7)
# --------------------------------------------------------------------------

def rope_theta(head_dim: int, base: float) -> np.ndarray:
    """theta_m = base ** (-2 m / d), m = 0 .. d/2 - 1, in float64."""
    if head_dim % 2:
        raise ValueError("head_dim must be even")
    m = np.arange(head_dim // 2, dtype=np.float64)
    return np.float64(base) ** (-(2.0 * m) / np.float64(head_dim))


def rope(x: np.ndarray, pos, theta: np.ndarray) -> np.ndarray:
    """Rotate x[n, ..., d] by the angles pos[n] * theta (pairs (m, m + d/2)).

    Negative positions rotate backwards, which is how the correction rotation
    Delta of [TS-M2] is expressed."""
    x = np.asarray(x, dtype=np.float64)
    pos = np.asarray(pos, dtype=np.float64)
    half = x.shape[-1] // 2
    ang = pos[:, None] * theta[None, :]                 # [n, d/2]
    shape = (ang.shape[0],) + (1,) * (x.ndim - 2) + (half,)
    c = np.cos(ang).reshape(shape)
    s = np.sin(ang).reshape(shape)
    x1 = x[..., :half]
    x2 = x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def _kv_map(num_q_heads: int, num_kv_heads: int, q_to_kv: Optional[Sequence[int]]):
    if q_to_kv is not None:
        return [int(x) for x in q_to_kv]
    if num_q_heads % num_kv_heads:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    per = num_q_heads // num_kv_heads
    return [h // per for h in range(num_q_heads)]


def _softmax_rows(s: np.ndarray, v: np.ndarray):
    """o = softmax(s) @ v and lse = log sum exp(s) over the last axis of s.
    Entries of s equal to -inf are excluded (causality)."""
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    z = np.sum(e, axis=-1, keepdims=True)
    o = (e @ v) / z
    lse = (m + np.log(z))[..., 0]
    return o, lse


# --------------------------------------------------------------------------
# prefill: distance-routed causal attention [TS-M1], [TS-M2]
# --------------------------------------------------------------------------

def prefill(q, k, v, *, w0: int, w_pretrained: int, rope_base: float,
            scale: Optional[float] = None, q_to_kv=None, rows=None,
            row_chunk: int = 256):
    """Bifocal causal attention of ONE sequence.

    q: [L, Hq, d], k, v: [L, Hkv, d] raw (pre-RoPE) projections, any float
    dtype (widened to float64).  rows: optional sorted query rows to evaluate
    (default: all).  Returns (o [len(rows), Hq, d], lse [Hq, len(rows)]) in
    float64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    L, Hq, d = q.shape
    Hkv = k.shape[1]
    rows = np.arange(L, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    n_rows = rows.shape[0]
    o_out = np.zeros((n_rows, Hq, d), dtype=np.float64)
    lse_out = np.zeros((Hq, n_rows), dtype=np.float64)
    if L == 0 or n_rows == 0:
        return o_out, lse_out
    scale = 1.0 / np.sqrt(d) if scale is None or scale <= 0 else float(scale)
    kv_of = _kv_map(Hq, Hkv, q_to_kv)

    G = group_size(L, w_pretrained)
    theta = rope_theta(d, rope_base)
    n_keys = int(rows.max()) + 1                       # keys any row can see
    kpos = np.arange(n_keys, dtype=np.int64)
    kb = rope(k[:n_keys], kpos, theta)                 # base keys, absolute positions
    kr = rope(k[:n_keys], remote_pos(kpos, G), theta)  # remote keys, f(j)
    qb = rope(q[rows], rows, theta)
    qr = rope(q[rows], remote_pos(rows, G), theta)

    for c0 in range(0, n_rows, row_chunk):
        r = rows[c0:c0 + row_chunk]
        nk = int(r.max()) + 1
        dist = r[:, None] - kpos[None, :nk]            # i - j
        local = (dist >= 0) & (dist < w0)              # R1
        visible = dist >= 0                            # causal
        for h in range(Hq):
            g = kv_of[h]
            s_base = qb[c0:c0 + row_chunk, h, :] @ kb[:nk, g, :].T
            s_rem = qr[c0:c0 + row_chunk, h, :] @ kr[:nk, g, :].T
            s = scale * np.where(local, s_base, s_rem)
            s = np.where(visible, s, -np.inf)
            o, lse = _softmax_rows(s, v[:nk, g, :])
            o_out[c0:c0 + row_chunk, h, :] = o
            lse_out[h, c0:c0 + row_chunk] = lse
    return o_out, lse_out


def prefill_varlen(q, k, v, cu_seqlens, *, w0, w_pretrained, rope_base,
                   scale=None, q_to_kv=None, rows_per_seq=None):
    """Packed independent sequences; positions restart at 0 and each sequence
    has its own G (R3).  rows_per_seq: optional list of row arrays (local to
    each sequence).  Returns lists of per-sequence (o, lse)."""
    outs = []
    for b in range(len(cu_seqlens) - 1):
        s0, s1 = int(cu_seqlens[b]), int(cu_seqlens[b + 1])
        rows = None if rows_per_seq is None else rows_per_seq[b]
        outs.append(prefill(q[s0:s1], k[s0:s1], v[s0:s1], w0=w0, w_pretrained=w_pretrained,
                            rope_base=rope_base, scale=scale, q_to_kv=q_to_kv, rows=rows))
    return outs


# --------------------------------------------------------------------------
# decode with the correction rotation Delta [TS-M2]
# --------------------------------------------------------------------------

def decode(q_base, k_cache, v_cache, L: int, *, w0: int, w_pretrained: int,
           rope_base: float, scale: Optional[float] = None, q_to_kv=None):
    """One generation step against a cache of base-RoPE keys.

    q_base: [Hq, d], already rotated by base RoPE at position i = L - 1 (R12).
    k_cache, v_cache: [>= L, Hkv, d]; row j holds the key rotated at absolute
    position j, and is used as given (never rewritten).
    Local keys (i - j < w0) score with the base vectors.  Remote keys score
    with the query and key moved to their aliased positions by the correction
    rotations Delta_q = f(i) - i and Delta_j = f(j) - j, G = group_size(L)
    (R4).  Returns (o [Hq, d], lse [Hq]) in float64.
    """
    q_base = np.asarray(q_base, dtype=np.float64)
    Hq, d = q_base.shape
    Hkv = k_cache.shape[1]
    if L <= 0:
        return np.zeros((Hq, d)), np.zeros((Hq,))
    scale = 1.0 / np.sqrt(d) if scale is None or scale <= 0 else float(scale)
    kv_of = _kv_map(Hq, Hkv, q_to_kv)
    K = np.asarray(k_cache[:L], dtype=np.float64)
    V = np.asarray(v_cache[:L], dtype=np.float64)

    G = group_size(L, w_pretrained)
    theta = rope_theta(d, rope_base)
    i = L - 1
    j = np.arange(L, dtype=np.int64)
    delta_q = int(remote_pos(i, G)) - i
    delta_k = remote_pos(j, G) - j
    q_rem = rope(q_base[None], np.array([delta_q]), theta)[0]   # R(f(i)) q
    k_rem = rope(K, delta_k, theta)                              # R(f(j)) k
    local = (i - j) < w0

    o = np.zeros((Hq, d))
    lse = np.zeros((Hq,))
    for h in range(Hq):
        g = kv_of[h]
        s_base = K[:, g, :] @ q_base[h]
        s_rem = k_rem[:, g, :] @ q_rem[h]
        s = scale * np.where(local, s_base, s_rem)
        oh, lh = _softmax_rows(s[None, :], V[:, g, :])
        o[h] = oh[0]
        lse[h] = lh[0]
    return o, lse
