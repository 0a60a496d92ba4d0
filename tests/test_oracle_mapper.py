"""Pins of the oracle's position mapper (Jet-Long technical summary,
Methodology item 1: group-size equation G and remote map f).

The oracle computes G with a ceiling division; it is checked against an exact
rational ceiling, a brute-force search for the minimal in-distribution G, the
hand-evaluated table in tests/golden/group_size.txt, and the invariants the
summary states (G = 1 inside the native window, remote positions stay inside
the pretraining grid, the compression is minimal)."""

import math
import os
import random
from fractions import Fraction

import numpy as np
import pytest

from oracle import group_size, remote_pos
from oracle.brute import group_size_search

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "group_size.txt")


def test_golden_table():
    n = 0
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        L, w, G = (int(x) for x in line.split())
        assert group_size(L, w) == G, (L, w)
        assert group_size_search(L, w) == G, (L, w)
        n += 1
    assert n >= 10


@pytest.mark.parametrize("w", [1, 2, 3, 7, 64, 4096, 32768])
def test_sweep_against_rational_ceiling(w):
    top = 1 << 17 if w >= 64 else 4000
    for L in range(0, top):
        G = group_size(L, w)
        assert G == max(1, math.ceil(Fraction(L, w))), (L, w)


@pytest.mark.parametrize("w", [1, 2, 3, 5, 64, 100])
def test_matches_minimal_search(w):
    for L in range(0, 2000):
        assert group_size(L, w) == group_size_search(L, w), (L, w)


def test_invariants_random_large():
    rng = random.Random(1234)
    for _ in range(20000):
        w = rng.choice([1, 2, 3, 64, 4096, 32768, rng.randint(1, 1 << 40)])
        L = rng.randint(0, 1 << 62)
        G = group_size(L, w)
        assert G >= 1
        # native window: G = 1 exactly when L <= w (base model recovered)
        assert (G == 1) == (L <= w)
        if L > 0:
            # in distribution: every aliased position f(x), x < L, is < w
            assert (L - 1) // G <= w - 1
            # minimal: one group fewer would leave the grid
            if G > 1:
                assert (L - 1) // (G - 1) >= w


def test_group_size_rejects_bad_args():
    with pytest.raises(ValueError):
        group_size(-1, 10)
    with pytest.raises(ValueError):
        group_size(10, 0)


def test_remote_pos_is_floor_division():
    x = np.arange(0, 10000)
    for G in (1, 2, 3, 4, 7):
        f = remote_pos(x, G)
        assert f.dtype == np.int64
        assert np.array_equal(f, np.array([xx // G for xx in range(10000)]))
        # G consecutive positions share one aliased position
        assert np.all(np.bincount(f)[:-1] == G)
    assert np.array_equal(remote_pos(x, 1), x)
