"""Host-side tests of the C ABI (no GPU): the library loads, exports every
declared entry point, computes G exactly, and rejects invalid arguments
before launching anything."""

import ctypes

import numpy as np
import pytest

import oracle
from jl_testutil import ensure_built, header_symbols

jl = ensure_built()
L = jl.lib()
JL_OK, JL_EINVAL, JL_EUNSUPPORTED, JL_ENOSPC = 0, -1, -2, -3
JL_MAX_SEQS = 64                 # include/jetlong.h


def test_exports_every_declared_symbol():
    names = header_symbols()
    assert {"jl_group_size", "jl_bifocal_prefill", "jl_bifocal_decode", "jl_last_error"} <= set(names)
    for n in names:
        assert hasattr(L, n), n


def test_group_size_matches_oracle():
    for w in (1, 3, 64, 4096, 32768):
        for n in list(range(0, 3000)) + [32767, 32768, 32769, 65536, 65537, 131072, 2**40 + 7, 2**62]:
            assert jl.group_size(n, w) == oracle.group_size(n, w), (n, w)


def test_group_size_rejects():
    assert L.jl_group_size(-1, 5) == JL_EINVAL
    assert L.jl_group_size(5, 0) == JL_EINVAL
    assert b"w_pretrained" in L.jl_last_error()


def _pf(fn="jl_bifocal_prefill", **kw):
    a = dict(q=None, k=None, v=None, o=None, lse=None, cu=None, nseq=1, T=256, Hq=4, Hkv=2, kvmap=None,
             d=128, dt=jl.BF16, w0=16, wpt=64, base=10000.0, scale=0.0, ws=None, nbytes=0)
    a.update(kw)
    n = ctypes.c_size_t(a["nbytes"])
    rc = getattr(L, fn)(a["q"], a["k"], a["v"], a["o"], a["lse"], a["cu"], a["nseq"], a["T"],
                              a["Hq"], a["Hkv"], a["kvmap"], a["d"], a["dt"], a["w0"], a["wpt"],
                              a["base"], a["scale"], a["ws"], ctypes.byref(n), None)
    return rc, n.value


def test_prefill_size_query():
    rc, n = _pf()
    assert rc == JL_OK and n > 0
    rc1, n1 = _pf(wpt=1000)          # G = 1: no remote copies
    assert rc1 == JL_OK and n1 < n
    rc0, n0 = _pf(T=0)
    assert rc0 == JL_OK and n0 == 0
    rc2, n2 = _pf(dt=jl.FP32, d=64)
    assert rc2 == JL_OK and n2 > 0


@pytest.mark.parametrize("kw,code", [
    (dict(T=-1), JL_EINVAL),
    (dict(Hq=3, Hkv=2), JL_EINVAL),
    (dict(Hq=0), JL_EINVAL),
    (dict(Hq=256, Hkv=2), JL_EUNSUPPORTED),
    (dict(d=96), JL_EUNSUPPORTED),
    (dict(d=64), JL_EUNSUPPORTED),            # bf16 path is built for d = 128
    (dict(dt=7), JL_EINVAL),
    (dict(w0=-1), JL_EINVAL),
    (dict(wpt=0), JL_EINVAL),
    (dict(base=0.0), JL_EINVAL),
    (dict(base=float("nan")), JL_EINVAL),
    (dict(nseq=0), JL_EINVAL),
    (dict(nseq=65, cu=(ctypes.c_int64 * 66)(*range(66)), T=65), JL_EUNSUPPORTED),
    (dict(nseq=2), JL_EINVAL),                # cu_seqlens missing
    (dict(nseq=2, cu=(ctypes.c_int64 * 3)(0, 300, 256)), JL_EINVAL),
    (dict(nseq=2, cu=(ctypes.c_int64 * 3)(1, 100, 256)), JL_EINVAL),
    (dict(nseq=2, cu=(ctypes.c_int64 * 3)(0, 100, 200)), JL_EINVAL),
    (dict(kvmap=(ctypes.c_int32 * 4)(0, 1, 2, 0)), JL_EINVAL),
    (dict(T=2**31), JL_EUNSUPPORTED),
])
def test_prefill_rejects(kw, code):
    rc, _ = _pf(**kw)
    assert rc == code, L.jl_last_error()
    assert L.jl_last_error()


def test_bf16_prefill_sequence_length_limit():
    # the bf16 pass kernels address one sequence's K/V rows with 31-bit byte
    # offsets: up to 2^23 - 64 tokens per sequence, checked on the host
    assert jl.BF16_MAX_SEQ_LEN == 2**23 - 64
    rc, n = _pf(T=jl.BF16_MAX_SEQ_LEN)
    assert rc == JL_OK and n > 0, L.jl_last_error()
    rc, _ = _pf(T=jl.BF16_MAX_SEQ_LEN + 1)
    assert rc == JL_EUNSUPPORTED and b"up to 8388544" in L.jl_last_error()
    T = jl.BF16_MAX_SEQ_LEN + 100
    rc, _ = _pf(T=T, nseq=2, cu=(ctypes.c_int64 * 3)(0, 100, T))
    assert rc == JL_OK, L.jl_last_error()              # both sequences within the limit
    rc, _ = _pf(T=T, nseq=2, cu=(ctypes.c_int64 * 3)(0, 99, T))
    assert rc == JL_EUNSUPPORTED and b"sequence 1" in L.jl_last_error()
    rc, _ = _pf(T=jl.BF16_MAX_SEQ_LEN + 1, dt=jl.FP32, d=64)
    assert rc == JL_OK, L.jl_last_error()              # the fp32 path has its own, larger limit


def test_fp32_prefill_sequence_length_limit():
    # one 64-lane workgroup per row: a sequence past 2^24 rows would exceed a
    # dispatch's 2^32 work-items, so the host refuses it before any launch
    assert jl.FP32_MAX_SEQ_LEN == 2**24
    rc, n = _pf(T=jl.FP32_MAX_SEQ_LEN, dt=jl.FP32, d=64)
    assert rc == JL_OK and n > 0, L.jl_last_error()
    rc, _ = _pf(T=jl.FP32_MAX_SEQ_LEN + 1, dt=jl.FP32, d=64)
    assert rc == JL_EUNSUPPORTED and b"fp32 prefill supports" in L.jl_last_error()
    T = jl.FP32_MAX_SEQ_LEN + 10
    rc, _ = _pf(T=T, nseq=2, cu=(ctypes.c_int64 * 3)(0, 10, T), dt=jl.FP32, d=64)
    assert rc == JL_OK, L.jl_last_error()


def test_prefill_workspace_too_small_is_enospc():
    rc, n = _pf()
    # a non-NULL workspace that is too small is refused before any device access
    rc2, _ = _pf(ws=0x1000, nbytes=n - 1, q=0x1000, k=0x1000, v=0x1000, o=0x1000)
    assert rc2 == JL_ENOSPC


def test_prefill_null_tensor_is_einval():
    rc, n = _pf()
    rc2, _ = _pf(ws=0x1000, nbytes=n)
    assert rc2 == JL_EINVAL


def test_disjoint_prefill_host_checks():
    # same workspace as the three-pass call, same argument checks, bf16 only
    rc, n = _pf()
    rcd, nd = _pf(fn="jl_bifocal_prefill_disjoint")
    assert rc == rcd == JL_OK and n == nd
    rc, _ = _pf(fn="jl_bifocal_prefill_disjoint", dt=jl.FP32, d=64)
    assert rc == JL_EUNSUPPORTED and b"bf16" in L.jl_last_error()
    assert _pf(fn="jl_bifocal_prefill_disjoint", Hq=3, Hkv=2)[0] == JL_EINVAL
    assert _pf(fn="jl_bifocal_prefill_disjoint", ws=0x1000, nbytes=n - 1, q=0x1000, k=0x1000, v=0x1000,
               o=0x1000)[0] == JL_ENOSPC
    assert _pf(fn="jl_bifocal_prefill_disjoint", ws=0x1000, nbytes=n)[0] == JL_EINVAL


def _pf_kc(kc, **kw):
    a = dict(q=None, k=None, v=None, o=None, lse=None, cu=None, nseq=1, T=256, Hq=4, Hkv=2, kvmap=None,
             d=128, dt=jl.BF16, w0=16, wpt=64, base=10000.0, scale=0.0, ws=None, nbytes=0)
    a.update(kw)
    n = ctypes.c_size_t(a["nbytes"])
    rc = L.jl_bifocal_prefill_kcache(a["q"], a["k"], a["v"], a["o"], a["lse"], kc, a["cu"], a["nseq"], a["T"],
                                     a["Hq"], a["Hkv"], a["kvmap"], a["d"], a["dt"], a["w0"], a["wpt"],
                                     a["base"], a["scale"], a["ws"], ctypes.byref(n), None)
    return rc, n.value


def test_kcache_prefill_host_checks():
    # the size query is the three-pass call's and ignores the cache pointer
    rc, n = _pf()
    assert _pf_kc(None) == (JL_OK, n) and _pf_kc(0x1000) == (JL_OK, n)
    assert _pf_kc(None, dt=jl.FP32, d=64) == _pf(dt=jl.FP32, d=64)
    # the argument checks of the three-pass call, before anything is launched
    assert _pf_kc(0x1000, Hq=3, Hkv=2)[0] == JL_EINVAL
    assert _pf_kc(0x1000, d=96)[0] == JL_EUNSUPPORTED
    ptrs = dict(ws=0x1000, nbytes=n, q=0x1000, k=0x1000, v=0x1000, o=0x1000)
    assert _pf_kc(0x1000, **dict(ptrs, nbytes=n - 1))[0] == JL_ENOSPC
    # a call that would launch needs the cache pointer, 16-byte aligned
    assert _pf_kc(None, **ptrs)[0] == JL_EINVAL and b"k_cache" in L.jl_last_error()
    assert _pf_kc(0x1008, **ptrs)[0] == JL_EINVAL and b"k_cache" in L.jl_last_error()
    # nothing to write: no tokens
    assert _pf_kc(None, T=0, ws=0x1000, nbytes=0) == (JL_OK, 0)


def _dec(**kw):
    a = dict(L=1000, Hq=32, Hkv=8, kvmap=None, d=128, dt=jl.BF16, w0=16, wpt=64, base=1e6, ws=None, nbytes=0)
    a.update(kw)
    n = ctypes.c_size_t(a["nbytes"])
    rc = L.jl_bifocal_decode(None, None, None, a["L"], None, None, a["Hq"], a["Hkv"], a["kvmap"], a["d"],
                             a["dt"], a["w0"], a["wpt"], a["base"], 0.0, a["ws"], ctypes.byref(n), None)
    return rc, n.value


def test_decode_size_query():
    rc, n = _dec()
    assert rc == JL_OK and n > 0
    rc, n = _dec(L=0)
    assert rc == JL_OK and n == 0
    assert _dec(L=131072)[1] >= _dec(L=1000)[1]


@pytest.mark.parametrize("kw,code", [
    (dict(L=-1), JL_EINVAL),
    (dict(dt=jl.FP32), JL_EUNSUPPORTED),
    (dict(d=64), JL_EUNSUPPORTED),
    (dict(Hq=12, Hkv=4), JL_EUNSUPPORTED),    # 3 q heads per kv head
    (dict(Hq=32, Hkv=16), JL_EUNSUPPORTED),
    (dict(Hq=4, Hkv=2, kvmap=(ctypes.c_int32 * 4)(0, 0, 0, 1)), JL_EUNSUPPORTED),
    (dict(w0=-3), JL_EINVAL),
    (dict(wpt=0), JL_EINVAL),
    (dict(L=2**31), JL_EUNSUPPORTED),
])
def test_decode_rejects(kw, code):
    rc, _ = _dec(**kw)
    assert rc == code, L.jl_last_error()


def test_decode_workspace_too_small_is_enospc():
    _, n = _dec()
    rc, _ = _dec(ws=0x1000, nbytes=n - 1)
    assert rc == JL_ENOSPC


def _decb(lens, row0=None, rows=None, **kw):
    a = dict(Hq=32, Hkv=8, kvmap=None, d=128, dt=jl.BF16, w0=16, wpt=64, base=1e6, ws=None, nbytes=0)
    a.update(kw)
    if row0 is None:
        row0 = [sum(lens[:b]) for b in range(len(lens))]
    if rows is None:
        rows = max([r + n for r, n in zip(row0, lens)] + [0])
    n = ctypes.c_size_t(a["nbytes"])
    arr = lambda v: (ctypes.c_int64 * max(1, len(v)))(*v)
    rc = L.jl_bifocal_decode_batch(None, None, None, rows, arr(row0), arr(lens), len(lens), None, None, a["Hq"],
                                   a["Hkv"], a["kvmap"], a["d"], a["dt"], a["w0"], a["wpt"], a["base"], 0.0,
                                   a["ws"], ctypes.byref(n), None)
    return rc, n.value


def test_decode_batch_size_query():
    # one sequence: the same workspace as the single-sequence call
    assert _decb([1000]) == _dec(L=1000)
    assert _decb([131072]) == _dec(L=131072)
    rc, n = _decb([5000, 0, 70000, 1])
    assert rc == JL_OK and n > 0
    assert _decb([0, 0]) == (JL_OK, 0)


@pytest.mark.parametrize("args,kw,code", [
    (([5, -1],), {}, JL_EINVAL),                         # negative length
    (([5, 2**31],), {}, JL_EUNSUPPORTED),
    (([5, 6], [0, -2]), {}, JL_EINVAL),                  # negative row0
    (([5, 6], [0, 5], 10), {}, JL_EINVAL),               # 5 + 6 rows past a cache of 10
    (([],), {}, JL_EINVAL),                              # no sequences
    (([1] * 65,), {}, JL_EUNSUPPORTED),                  # more than JL_MAX_SEQS
    (([5],), dict(dt=jl.FP32), JL_EUNSUPPORTED),
    (([5],), dict(Hq=12, Hkv=4), JL_EUNSUPPORTED),
    (([5],), dict(w0=-1), JL_EINVAL),
])
def test_decode_batch_rejects(args, kw, code):
    rc, _ = _decb(*args, **kw)
    assert rc == code, L.jl_last_error()
    assert L.jl_last_error()


def test_decode_batch_overlapping_rows_and_null_pointers():
    rc, n = _decb([100, 100], row0=[0, 50], rows=150)    # shared cache rows are allowed
    assert rc == JL_OK and n > 0
    assert _decb([100, 100], row0=[0, 50], rows=150, ws=0x1000, nbytes=n)[0] == JL_EINVAL
    assert _decb([100, 100], row0=[0, 50], rows=150, ws=0x1000, nbytes=n - 1)[0] == JL_ENOSPC
    assert L.jl_bifocal_decode_batch(None, None, None, -1, None, None, 1, None, None, 32, 8, None, 128, jl.BF16,
                                     16, 64, 1e6, 0.0, None, ctypes.byref(ctypes.c_size_t(0)), None) == JL_EINVAL


def test_rope_rows_rejects_before_launch():
    f = L.jl_rope_rows
    assert f(None, None, 0, 2, 128, jl.BF16, 0, 1e4, None) == JL_OK            # empty: no-op
    assert f(None, None, -1, 2, 128, jl.BF16, 0, 1e4, None) == JL_EINVAL
    assert f(None, None, 4, 2, 128, jl.BF16, -1, 1e4, None) == JL_EINVAL
    assert f(None, None, 4, 0, 128, jl.BF16, 0, 1e4, None) == JL_EINVAL
    assert f(None, None, 4, 2, 127, jl.BF16, 0, 1e4, None) == JL_EUNSUPPORTED
    assert f(None, None, 4, 2, 256, jl.BF16, 0, 1e4, None) == JL_EUNSUPPORTED
    assert f(None, None, 4, 2, 128, jl.BF16, 2**31 - 2, 1e4, None) == JL_EUNSUPPORTED
    assert f(None, None, 4, 2, 128, jl.BF16, 0, -1.0, None) == JL_EINVAL
    assert f(None, None, 4, 2, 128, 7, 0, 1e4, None) == JL_EINVAL
    assert f(None, None, 4, 2, 128, jl.BF16, 0, 1e4, None) == JL_EINVAL       # null pointers
    assert b"device pointers" in L.jl_last_error()


def _plan(lens, cus):
    nsub, nwg = ctypes.c_int32(), ctypes.c_int32()
    arr = (ctypes.c_int64 * len(lens))(*lens)
    rc = L.jl_test_decode_plan(arr, len(lens), cus, ctypes.byref(nsub), ctypes.byref(nwg))
    assert rc == JL_OK, L.jl_last_error()
    return nsub.value, nwg.value


def test_decode_plan_follows_the_compute_unit_count():
    """The split plan fills one round of the device's compute units: the
    smallest 64-key sub-chunk count whose workgroups fit one per CU.  A full
    MI355X (256 CUs) and its partition modes (128, 64, 32 CUs) each get
    their own plan."""
    for cus, nsub in ((256, 8), (128, 16), (64, 32), (32, 64)):
        assert _plan([131072], cus) == (nsub, cus), cus
    # 32769 keys = 513 sub-chunks: 171 workgroups of 3 on 256 CUs, 65 of 8 on 80 CUs
    assert _plan([32769], 256) == (3, 171)
    assert _plan([32769], 80) == (7, 74)
    # one key per CU at most: small caches take one sub-chunk per workgroup
    assert _plan([100], 256) == (1, 2)
    # a batch shares one plan across its sequences
    nsub, nwg = _plan([131072, 65536, 1], 256)
    assert nwg <= 256 and _plan([131072, 65536, 1], 128)[1] <= 128
    for cus in (7, 100, 304):
        nsub, nwg = _plan([131072, 12345], cus)
        assert nwg <= cus
        assert nsub == 1 or sum(-(-n // (64 * (nsub - 1))) for n in (131072, 12345)) > cus
    bad = ctypes.c_int32()
    assert L.jl_test_decode_plan((ctypes.c_int64 * 1)(5), 1, 0, ctypes.byref(bad), ctypes.byref(bad)) == JL_EINVAL


def test_decode_prefix_sums_support_the_kernels_search():
    """The split kernel finds a workgroup's sequence by counting the sequence
    starts after the first that lie at or before it (one ballot), and both
    decode kernels read the total workgroup count from the last prefix-sum
    slot.  Both rest on the plan's prefix sums: they never decrease, and
    every entry from the sequence count on holds the total.  The count must
    equal a linear search over the starts for every workgroup, also with
    sequences of no keys (which own no workgroups)."""
    rng = np.random.default_rng(7)
    cases = [[131072], [0, 5, 0], [32769, 1, 64, 65], [0] * 7 + [100],
             [int(x) for x in rng.integers(0, 200000, size=64)],
             [int(x) for x in rng.integers(0, 3, size=40)]]
    for lens in cases:
        for cus in (256, 80, 7):
            arr = (ctypes.c_int64 * len(lens))(*lens)
            wb = (ctypes.c_int32 * (JL_MAX_SEQS + 1))()
            assert L.jl_test_decode_prefix(arr, len(lens), cus, wb) == JL_OK, L.jl_last_error()
            wb = list(wb)
            nsub, nwg = _plan(lens, cus)
            n = len(lens)
            assert wb[0] == 0 and all(wb[i] <= wb[i + 1] for i in range(JL_MAX_SEQS))
            assert all(wb[i] == nwg for i in range(n, JL_MAX_SEQS + 1))
            for b in range(n):                   # each sequence owns its keys' workgroups
                assert wb[b + 1] - wb[b] == -(-lens[b] // (64 * nsub))
            for w in range(nwg):
                lin = 0
                while lin + 1 < n and w >= wb[lin + 1]:
                    lin += 1
                cnt = sum(1 for k in range(1, min(n, 65)) if w >= wb[k])
                assert cnt == lin and lens[lin] > 0, (lens, cus, w)
    bad = (ctypes.c_int32 * (JL_MAX_SEQS + 1))()
    assert L.jl_test_decode_prefix((ctypes.c_int64 * 1)(-1), 1, 256, bad) == JL_EINVAL


def test_device_shape_default_without_a_device():
    """On a host without a GPU the library plans for the full MI355X shape;
    on a GPU the shape is read from the device (checked by the GPU tests)."""
    import torch
    cus, xcds = ctypes.c_int32(), ctypes.c_int32()
    assert L.jl_test_device_shape(ctypes.byref(cus), ctypes.byref(xcds)) == JL_OK
    if not torch.cuda.is_available():
        assert (cus.value, xcds.value) == (256, 8)
    else:
        assert cus.value >= 1 and 1 <= xcds.value <= cus.value


def test_decode_workspace_never_shrinks_as_L_grows():
    """The plan's workgroup count falls where the sub-chunk count per
    workgroup steps up (32767 keys: 256 workgroups of 2 sub-chunks, 32771
    keys: 171 of 3), but the workspace size does not: a workspace sized for
    the longest step of a generation loop serves every shorter one."""
    sizes = [jl.decode_workspace_bytes(L, 32, 8) for L in range(32700, 32900)]
    assert all(a <= b for a, b in zip(sizes, sizes[1:]))
    Ls = [0, 1, 63, 64, 65, 1000, 16383, 16384, 16385, 40000, 131072, 2**22, 2**24, 2**25, 2**26 + 1]
    sizes = [jl.decode_workspace_bytes(L, 32, 8) for L in Ls]
    assert all(a <= b for a, b in zip(sizes, sizes[1:])), sizes
    b1 = jl.decode_batch_workspace_bytes([32767, 100], 32, 8)
    b2 = jl.decode_batch_workspace_bytes([32771, 100], 32, 8)
    assert b1 <= b2


def _na(L=1000, Hq=32, Hkv=8, ptr=None):
    return L_.jl_bifocal_decode_noalloc(ptr, ptr, ptr, L, ptr, None, Hq, Hkv, None, 128, jl.BF16, 16, 64, 1e6, 0.0,
                                        None)


L_ = L


def test_decode_noalloc_host_checks():
    """The no-allocation decode validates like jl_bifocal_decode, refuses a
    call whose partials exceed its scratch, and does nothing for L = 0, all
    before it touches a device."""
    assert jl.DECODE_SCRATCH_BYTES == 256 * 32 * 130 * 4
    assert _na(L=0) == JL_OK
    assert _na(Hq=3) == JL_EINVAL
    assert _na(L=-1) == JL_EINVAL
    assert _na(Hq=64, L=131072) == JL_EUNSUPPORTED and b"no-allocation scratch" in L.jl_last_error()
    assert _na() == JL_EINVAL and b"device pointers" in L.jl_last_error()
    # within the scratch: the workspace the two-call protocol would ask for
    for Lx in (1, 4097, 131072, 2**24):
        assert jl.decode_workspace_bytes(Lx, 32, 8) <= jl.DECODE_SCRATCH_BYTES
