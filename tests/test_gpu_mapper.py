"""Device build of the position mapper and angle formation, bit for bit
(G, f) and within fp32 rounding (angles), against exact integers and fp64
(technical summary, Methodology item 1: group-size equation and remote map)."""

import math
import sys

import numpy as np
import pytest

import oracle
from jl_testutil import gpu_or_skip

pytestmark = pytest.mark.gpu


def test_device_group_size_exact():
    jl, torch = gpu_or_skip()
    Ls = list(range(0, 5000)) + [32767, 32768, 32769, 65535, 65536, 65537, 98304, 98305, 131071,
                                 131072, 131073, 2**31 - 1, 2**40 + 3, 2**62 + 11]
    for w in (1, 2, 3, 64, 4096, 32768):
        Lt = torch.tensor(Ls, dtype=torch.int64, device="cuda")
        Gt = torch.empty_like(Lt)
        rc = jl.lib().jl_test_group_size_device(Lt.data_ptr(), len(Ls), w, Gt.data_ptr(), None)
        assert rc == 0
        torch.cuda.synchronize()
        got = Gt.cpu().tolist()
        assert got == [oracle.group_size(n, w) for n in Ls], w


@pytest.mark.parametrize("G", [1, 2, 3, 4, 5, 7])
def test_device_remote_pos_exact(G):
    jl, torch = gpu_or_skip()
    n = 1 << 18
    for x0 in (0, 2**31 - 1 - n):
        f = torch.empty(n, dtype=torch.int32, device="cuda")
        assert jl.lib().jl_test_remote_pos_device(x0, n, G, f.data_ptr(), None) == 0
        torch.cuda.synchronize()
        want = oracle.remote_pos(np.arange(x0, x0 + n, dtype=np.int64), G)
        assert np.array_equal(f.cpu().numpy().astype(np.int64), want)


def test_device_angles_accurate_at_long_positions():
    """cos/sin of p * theta_m at positions up to 2^31 - 1 (and negative, the
    Delta corrections) stay within 2e-6 of fp64 for every frequency."""
    jl, torch = gpu_or_skip()
    rng = np.random.default_rng(0)
    pos = np.concatenate([np.arange(-5000, 5000), rng.integers(-2**31 + 1, 2**31 - 1, 20000),
                          [131071, -98303, 2**31 - 1]]).astype(np.int32)
    pt = torch.from_numpy(pos).cuda()
    c = torch.empty(len(pos), dtype=torch.float32, device="cuda")
    s = torch.empty_like(c)
    worst = 0.0
    for d, base in ((128, 1e6), (64, 1e4)):
        th = oracle.rope_theta(d, base)
        for m in range(d // 2):
            assert jl.lib().jl_test_rope_angles_device(pt.data_ptr(), len(pos), m, d, base,
                                                       c.data_ptr(), s.data_ptr(), None) == 0
            torch.cuda.synchronize()
            ang = pos.astype(np.float64) * th[m]
            err = max(np.abs(c.cpu().numpy() - np.cos(ang)).max(), np.abs(s.cpu().numpy() - np.sin(ang)).max())
            worst = max(worst, err)
    assert worst < 2e-6, worst


def test_device_shape_matches_the_runtime():
    """The library plans with the device's own compute-unit count (decode's
    one-round split) and XCD count (prefill's per-XCD head groups)."""
    import ctypes
    jl, torch = gpu_or_skip()
    cus, xcds = ctypes.c_int32(), ctypes.c_int32()
    assert jl.lib().jl_test_device_shape(ctypes.byref(cus), ctypes.byref(xcds)) == 0
    props = torch.cuda.get_device_properties(0)
    print(f"[shape] {props.name}: {cus.value} CUs, {xcds.value} XCDs", file=sys.stderr, flush=True)
    assert cus.value == props.multi_processor_count
    assert 1 <= xcds.value <= cus.value and cus.value % xcds.value == 0
