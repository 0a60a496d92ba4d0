"""Parity of the HIP bifocal decode step with the fp64 oracle, including the
steps that cross a G boundary, and a check that the cache is never written
(technical summary, Methodology item 2: correction rotation Delta applied to
the query and the cached keys in registers)."""

import sys

import numpy as np
import pytest

import oracle
import workloads as W
from jl_testutil import BF16_LSE_RTOL, BF16_O_ATOL, gpu_or_skip, lse_rel_err, max_abs

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _decode_case(jl, torch, L, Hq, Hkv, w0, wpt, base, seed, L_cap=None, q_to_kv=None):
    cfg = W.DecodeConfig("case", Hq, Hkv, 128, L, w0, wpt, base, seed)
    q, kc, vc = W.make_decode_inputs(cfg, L_cap=L_cap)
    _say(f"[decode] L={L} Hq={Hq} Hkv={Hkv} w0={w0} wpt={wpt} cap={kc.shape[0]} seed={seed}")
    qd, kd, vd = q.cuda(), kc.cuda(), vc.cuda()
    k_before, v_before = kd.clone(), vd.clone()
    o, lse = jl.decode(qd, kd, vd, L, w0=w0, w_pretrained=wpt, rope_base=base, q_to_kv=q_to_kv)
    torch.cuda.synchronize()
    # the cache is never written: every bit of both caches is unchanged
    assert torch.equal(kd.view(torch.int16), k_before.view(torch.int16))
    assert torch.equal(vd.view(torch.int16), v_before.view(torch.int16))
    oo, ll = oracle.decode(q.double().numpy(), kc[:L].double().numpy(), vc[:L].double().numpy(), L,
                           w0=w0, w_pretrained=wpt, rope_base=base, q_to_kv=q_to_kv)
    og, lg = o.float().cpu().numpy(), lse.cpu().numpy()
    e_o, e_l = max_abs(og, oo), lse_rel_err(lg, ll)
    _say(f"[decode] L={L}: max|do|={e_o:.3e} lse rel={e_l:.3e}")
    assert e_o <= BF16_O_ATOL
    assert e_l <= BF16_LSE_RTOL
    return og, lg


@pytest.mark.parametrize("L", W.DECODE_LENGTHS)
def test_qwen3_8b_decode_lengths(L):
    """32 q / 8 kv heads, d = 128, w0 = 4096, w_pretrained = 32768, at 16K,
    32K, 32769 (G 1 -> 2), 64K, 65537 (G 2 -> 3) and 128K (G = 4)."""
    jl, torch = gpu_or_skip()
    _decode_case(jl, torch, L, 32, 8, 4096, 32768, 1e6, seed=L)


@pytest.mark.parametrize("L,Hq,Hkv,w0,wpt", [
    (1, 4, 2, 4, 8),
    (63, 4, 2, 10, 16),          # one partial sub-chunk, G = 4
    (65, 8, 8, 64, 16),          # sub-chunk edge, G = 5
    (300, 8, 2, 0, 100),         # w0 = 0: every key remote
    (300, 8, 2, 500, 100),       # w0 >= L: every key local
    (1000, 16, 2, 100, 2000),    # G = 1
    (4097, 2, 2, 1, 1024),       # w0 = 1
    (5000, 32, 8, 333, 1200),    # G = 5, ragged
    (777, 3, 3, 100, 256),       # odd kv-head count: a wave with one kv head
    (129, 8, 1, 20, 40),         # one kv head, 8 q heads per kv head, G = 4
    (2000, 64, 8, 200, 600),     # 64 q heads, G = 4
    # the angle table steps over 8 keys by floor(8 / G) - 8 or that plus one:
    # G = 8 (a step of 1), G = 9 and larger (a step of 0)
    (2000, 4, 2, 50, 250),       # G = 8
    (2000, 4, 2, 50, 223),       # G = 9
    (3000, 8, 2, 100, 130),      # G = 24
    (70000, 8, 2, 4096, 1000),   # G = 70, many sub-chunks per workgroup
])
def test_small_decode_cases(L, Hq, Hkv, w0, wpt):
    jl, torch = gpu_or_skip()
    _decode_case(jl, torch, L, Hq, Hkv, w0, wpt, 1e4, seed=L + 7, L_cap=L + 37)


def test_head_map():
    jl, torch = gpu_or_skip()
    _decode_case(jl, torch, 700, 4, 2, 50, 256, 1e4, seed=3, q_to_kv=[1, 0, 0, 1])


def test_decode_equals_last_prefill_row():
    """decode(L) on the cache of base-rotated keys equals the last row of the
    bifocal prefill at L: the oracle's last row, and the library's.  The
    decode runs twice, on a cache rotated on the host (fp64, rounded to bf16)
    and on the cache the library's prefill writes; each result is checked
    against the oracle at the bf16 bars, and against the library's own
    prefill row at twice them (two results each within the bar of the
    oracle)."""
    jl, torch = gpu_or_skip()
    L, Hq, Hkv, w0, wpt, base = 1500, 8, 2, 200, 400, 1e6   # G = 4
    g = torch.Generator("cpu").manual_seed(11)
    q = torch.randn((L, Hq, 128), generator=g).bfloat16()
    k = torch.randn((L, Hkv, 128), generator=g).bfloat16()
    v = torch.randn((L, Hkv, 128), generator=g).bfloat16()
    kc_lib = torch.empty((L, Hkv, 128), dtype=torch.bfloat16, device="cuda")
    o_p, lse_p = jl.prefill(q.cuda(), k.cuda(), v.cuda(), w0=w0, w_pretrained=wpt, rope_base=base,
                            k_cache_out=kc_lib)
    # cache and query rotated at absolute positions (fp64 on the host, rounded to bf16)
    th = oracle.rope_theta(128, base)
    kc = torch.from_numpy(oracle.rope(k.double().numpy(), np.arange(L), th)).bfloat16()
    qb = torch.from_numpy(oracle.rope(q[L - 1:L].double().numpy(), np.array([L - 1]), th)[0]).bfloat16()
    o_ref, lse_ref = oracle.prefill(q.double().numpy(), k.double().numpy(), v.double().numpy(),
                                    w0=w0, w_pretrained=wpt, rope_base=base, rows=[L - 1])
    for name, cache in (("host-rotated cache", kc.cuda()), ("prefill-written cache", kc_lib)):
        o_d, lse_d = jl.decode(qb.cuda(), cache, v.cuda(), L, w0=w0, w_pretrained=wpt, rope_base=base)
        torch.cuda.synchronize()
        od, ld = o_d.float().cpu().numpy(), lse_d.cpu().numpy()
        e_o, e_l = max_abs(od, o_ref[0]), lse_rel_err(ld, lse_ref[:, 0])
        print(f"[decode] {name}: vs oracle max|do|={e_o:.3e} lse rel={e_l:.3e}")
        assert e_o <= BF16_O_ATOL and e_l <= BF16_LSE_RTOL
        assert max_abs(od, o_p[L - 1].float().cpu().numpy()) <= 2 * BF16_O_ATOL
        assert lse_rel_err(ld, lse_p[:, L - 1].cpu().numpy()) <= 2 * BF16_LSE_RTOL
    # the library's prefill row itself, against the oracle
    assert max_abs(o_p[L - 1].float().cpu().numpy(), o_ref[0]) <= BF16_O_ATOL
    assert lse_rel_err(lse_p[:, L - 1].cpu().numpy(), lse_ref[:, 0]) <= BF16_LSE_RTOL


def test_empty_cache_is_noop():
    jl, torch = gpu_or_skip()
    q = torch.zeros((4, 128), dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros((8, 2, 128), dtype=torch.bfloat16, device="cuda")
    o, lse = jl.decode(q, kc, kc, 0, w0=4, w_pretrained=8, rope_base=1e4)
    torch.cuda.synchronize()
    assert o.shape == (4, 128)


@pytest.mark.parametrize("L", [65537, 131072])
def test_repeated_calls_are_bitwise_identical(L):
    """A wave reads a sub-chunk's angle table only after every wave of the
    workgroup has written its share, so identical calls give identical bits
    (regression: a shared-total progress counter once let fast waves read a
    table that slow waves were still filling)."""
    jl, torch = gpu_or_skip()
    cfg = W.decode_8b(L)
    q, kc, vc = W.make_decode_inputs(cfg)
    qd, kd, vd = q.cuda(), kc.cuda(), vc.cuda()
    kw = dict(w0=cfg.w0, w_pretrained=cfg.w_pretrained, rope_base=cfg.rope_base)
    o0, l0 = jl.decode(qd, kd, vd, L, **kw)
    for _ in range(4):
        o, l = jl.decode(qd, kd, vd, L, **kw)
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), o0.view(torch.int16))
        assert torch.equal(l, l0)
