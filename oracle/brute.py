"""Pure-Python brute force of bifocal attention for tiny inputs.

TEST INFRASTRUCTURE ONLY (see ``oracle/jetlong.py``).  Written with the math
module and explicit loops, independently of numpy, to pin the vectorised
oracle.  RoPE is built here as an explicit d x d block-rotation matrix that
rotates the plane of coordinates (m, m + d/2) by pos * theta_m (reading R7),
and G is found by searching for the smallest integer group that keeps every
aliased position inside the pretraining grid (Jet-Long technical summary,
Methodology item 1: the minimum compression that keeps remote angles in
distribution), rather than by the ceiling formula.
"""

from __future__ import annotations

import math


def group_size_search(L, w_pretrained):
    """Smallest G >= 1 with floor((L - 1) / G) <= w_pretrained - 1."""
    G = 1
    while L > 0 and (L - 1) // G > w_pretrained - 1:
        G += 1
    return G


def rotation_matrix(d, pos, base):
    R = [[0.0] * d for _ in range(d)]
    half = d // 2
    for m in range(half):
        th = base ** (-(2.0 * m) / d)
        a = pos * th
        c, s = math.cos(a), math.sin(a)
        # plane (m, m + half): x_m' = c x_m - s x_{m+h}; x_{m+h}' = s x_m + c x_{m+h}
        R[m][m] = c
        R[m][m + half] = -s
        R[m + half][m] = s
        R[m + half][m + half] = c
    return R


def matvec(R, x):
    return [sum(R[a][b] * x[b] for b in range(len(x))) for a in range(len(R))]


def dot(a, b):
    return sum(x * y for x, y in zip(a, b))


def prefill_brute(q, k, v, w0, w_pretrained, base, scale=None):
    """q, k, v: nested lists [L][d] for ONE head.  Returns (o [L][d], lse [L])."""
    L = len(q)
    d = len(q[0]) if L else 0
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    G = group_size_search(L, w_pretrained)
    o, lse = [], []
    for i in range(L):
        scores = []
        for j in range(i + 1):
            if i - j < w0:
                qi = matvec(rotation_matrix(d, i, base), q[i])
                kj = matvec(rotation_matrix(d, j, base), k[j])
            else:
                qi = matvec(rotation_matrix(d, i // G, base), q[i])
                kj = matvec(rotation_matrix(d, j // G, base), k[j])
            scores.append(scale * dot(qi, kj))
        m = max(scores)
        w = [math.exp(s - m) for s in scores]
        z = sum(w)
        o.append([sum(w[j] * v[j][c] for j in range(i + 1)) / z for c in range(d)])
        lse.append(m + math.log(z))
    return o, lse


def decode_brute(q_base, K, V, L, w0, w_pretrained, base, scale=None):
    """One head.  q_base rotated at position L - 1; K[j] rotated at j.
    Remote keys are first un-rotated to raw form and re-rotated at their
    aliased position, and likewise the query: an explicit version of the
    correction rotation."""
    d = len(q_base)
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    G = group_size_search(L, w_pretrained)
    i = L - 1
    Rt = lambda p: [list(r) for r in zip(*rotation_matrix(d, p, base))]   # inverse = transpose
    q_raw = matvec(Rt(i), q_base)
    scores = []
    for j in range(L):
        if i - j < w0:
            scores.append(scale * dot(q_base, K[j]))
        else:
            k_raw = matvec(Rt(j), K[j])
            qi = matvec(rotation_matrix(d, i // G, base), q_raw)
            kj = matvec(rotation_matrix(d, j // G, base), k_raw)
            scores.append(scale * dot(qi, kj))
    m = max(scores)
    w = [math.exp(s - m) for s in scores]
    z = sum(w)
    o = [sum(w[j] * V[j][c] for j in range(L)) / z for c in range(d)]
    return o, m + math.log(z)
