"""Host-side pieces of bench.py: the FLOP counts it divides by, checked against
pair counts taken one row at a time, and the one-GPU guard."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _pairs(L, w0):
    causal = sum(i + 1 for i in range(L))
    window = sum(min(i + 1, w0) for i in range(L))
    far = sum(max(0, i + 1 - w0) for i in range(L))
    return causal, window, far


@pytest.mark.parametrize("L,w0", [(1, 1), (7, 3), (300, 37), (300, 300), (300, 1000), (1000, 0), (4096, 128)])
def test_prefill_flops_match_pair_counts(L, w0):
    Hq, d = 3, 128
    causal, window, _ = _pairs(L, w0)
    F3, Fc = bench.prefill_flops(L, Hq, d, w0)
    assert Fc == 4 * d * Hq * causal
    assert F3 == 4 * d * Hq * (causal + 2 * window)


@pytest.mark.parametrize("L,w0", [(300, 37), (300, 200), (300, 400), (1000, 1), (131, 128), (5000, 4096)])
def test_far_flops_match_pair_counts(L, w0):
    Hq, d = 2, 128
    far_rows = sum(max(0, i + 1 - w0) for i in range(128, L))   # rows >= 128 of the 256-row kernels
    assert bench.far_flops(L, Hq, d, w0) == 4 * d * Hq * far_rows
    # window + far = causal over the same rows
    win_rows = sum(min(i + 1, w0) for i in range(128, L))
    assert win_rows + far_rows == sum(i + 1 for i in range(128, L))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_varlen_flops_are_the_sum_over_sequences():
    lens = [5, 300, 0, 1, 77]
    Hq, d, w0 = 2, 64, 40
    f3, fc = bench.prefill_flops_varlen(lens, Hq, d, w0)
    causal = sum(_pairs(n, w0)[0] for n in lens)
    window = sum(_pairs(n, w0)[1] for n in lens)
    assert fc == 4 * d * Hq * causal and f3 == 4 * d * Hq * (causal + 2 * window)
    for L in (0, 1, 39, 40, 41, 500):
        assert bench.window_pairs(L, w0) == _pairs(L, w0)[1]
