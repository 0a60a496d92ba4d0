"""Planted mistakes in the oracle must be caught by its pins.

Each case rewrites one line of ``oracle/jetlong.py`` in memory (a dropped
term, a wrong sign, an off-by-one window edge, a wrong grid), loads the
mutant as a separate module and checks that the independent brute force no
longer agrees.  Nothing on disk changes and nothing here touches a GPU."""

import os
import types

import numpy as np
import pytest

from oracle import brute

SRC = os.path.join(os.path.dirname(os.path.dirname(__file__)), "oracle", "jetlong.py")

MUTANTS = {
    "rope_sign": ("x2 * c + x1 * s], axis=-1)", "x2 * c - x1 * s], axis=-1)"),
    "rope_pairs": ("x1 * c - x2 * s, x2", "x1 * c + x2 * s, x2"),
    "window_edge": ("local = (dist >= 0) & (dist < w0)", "local = (dist >= 0) & (dist <= w0)"),
    "group_floor": ("ceil_div = -((-L) // w_pretrained)", "ceil_div = L // w_pretrained"),
    "query_not_aliased": ("qr = rope(q[rows], remote_pos(rows, G), theta)", "qr = rope(q[rows], rows, theta)"),
    "theta_exponent": ("(-(2.0 * m) / np.float64(head_dim))", "(-(1.0 * m) / np.float64(head_dim))"),
    "decode_delta_sign": ("delta_q = int(remote_pos(i, G)) - i", "delta_q = i - int(remote_pos(i, G))"),
    "decode_window": ("local = (i - j) < w0", "local = (i - j) <= w0"),
    "lse_drop_max": ("lse = (m + np.log(z))[..., 0]", "lse = (np.log(z))[..., 0]"),
}


def _load_mutant(name):
    old, new = MUTANTS[name]
    text = open(SRC).read()
    assert text.count(old) == 1, name
    mod = types.ModuleType("oracle_mutant_" + name)
    mod.__dict__["__name__"] = mod.__name__
    exec(compile(text.replace(old, new), SRC + ":" + name, "exec"), mod.__dict__)
    return mod


def _prefill_disagrees(m):
    rng = np.random.default_rng(0)
    L, d, w0, w_pt, base = 24, 8, 5, 7, 100.0
    q, k, v = (rng.standard_normal((L, 1, d)) for _ in range(3))
    try:
        o, lse = m.prefill(q, k, v, w0=w0, w_pretrained=w_pt, rope_base=base)
    except Exception:
        return True
    ob, lb = brute.prefill_brute(q[:, 0].tolist(), k[:, 0].tolist(), v[:, 0].tolist(), w0, w_pt, base)
    return not (np.allclose(o[:, 0], ob, atol=1e-9) and np.allclose(lse[0], lb, atol=1e-9))


def _decode_disagrees(m):
    rng = np.random.default_rng(1)
    L, d, w0, w_pt, base = 20, 8, 4, 6, 100.0
    K = []
    for j in range(L):
        K.append(brute.matvec(brute.rotation_matrix(d, j, base), list(rng.standard_normal(d))))
    V = rng.standard_normal((L, d))
    qb = brute.matvec(brute.rotation_matrix(d, L - 1, base), list(rng.standard_normal(d)))
    try:
        o, lse = m.decode(np.array([qb]), np.array(K)[:, None], V[:, None], L, w0=w0,
                          w_pretrained=w_pt, rope_base=base)
    except Exception:
        return True
    ob, lb = brute.decode_brute(qb, K, V.tolist(), L, w0, w_pt, base)
    return not (np.allclose(o[0], ob, atol=1e-9) and np.allclose(lse[0], lb, atol=1e-9))


def test_unmutated_oracle_agrees():
    import oracle.jetlong as orig
    assert not _prefill_disagrees(orig)
    assert not _decode_disagrees(orig)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    m = _load_mutant(name)
    assert _prefill_disagrees(m) or _decode_disagrees(m), name
