"""Streaming prefill -> decode chain on the device (technical summary,
Methodology item 2: the cache holds keys rotated by base RoPE at their
absolute positions; generation applies the correction rotation on the fly and
never rewrites the cache, also when the length crosses a G boundary).

The prompt's cache is written by the prefill itself (`jl_bifocal_prefill_kcache`,
checked bitwise against `jl_rope_rows`), extended with the row rotation,
the decode loop appends one token per step across
L = 32768 -> 32769 (G 1 -> 2), and every step is checked against the last row
of the fp64 oracle prefill at that length and against the library's own
prefill."""

import sys

import numpy as np
import pytest

import oracle
from jl_testutil import BF16_LSE_RTOL, BF16_O_ATOL, gpu_or_skip, lse_rel_err, max_abs

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.mark.parametrize("pos0", [0, 32700, 131000, 2**31 - 300])
def test_rope_rows_matches_oracle(pos0):
    jl, torch = gpu_or_skip()
    g = torch.Generator("cpu").manual_seed(pos0 % 1000 + 5)
    n, H, d, base = 300, 3, 128, 1e6
    x = torch.randn((n, H, d), generator=g)
    theta = oracle.rope_theta(d, base)
    ref = oracle.rope(x.double().numpy(), np.arange(pos0, pos0 + n), theta)
    _say(f"[rope] pos0={pos0}")
    # fp32: the rotation itself, against the fp64 angles
    y32 = jl.rope_rows(x.cuda(), pos0, rope_base=base).cpu().double().numpy()
    assert max_abs(y32, ref) <= 1e-5
    # bf16: input and output rounded to bf16, math in fp32
    xb = x.to(torch.bfloat16)
    refb = oracle.rope(xb.double().numpy(), np.arange(pos0, pos0 + n), theta)
    yb = jl.rope_rows(xb.cuda(), pos0, rope_base=base)
    err = np.abs(yb.cpu().double().numpy() - refb)
    assert np.all(err <= 2.0 ** -8 * np.abs(refb) + 1e-6)
    # in place gives the same bits
    xi = xb.cuda()
    jl.rope_rows(xi, pos0, rope_base=base, out=xi)
    assert torch.equal(xi.view(torch.int16), yb.view(torch.int16))
    # a rotation keeps every pair's norm
    half = d // 2
    nx = x[..., :half] ** 2 + x[..., half:] ** 2
    ny = torch.from_numpy(y32[..., :half] ** 2 + y32[..., half:] ** 2)
    assert torch.allclose(nx.double(), ny, rtol=1e-5, atol=1e-6)


def test_rope_rows_alternating_bases_and_dims():
    """The library keeps the last frequency table it built (per host thread),
    keyed by head_dim and base: calls that alternate both must each get their
    own table, checked against the fp64 oracle (a stale table would rotate
    by the wrong angles)."""
    jl, torch = gpu_or_skip()
    g = torch.Generator("cpu").manual_seed(11)
    pos0, n, H = 4000, 64, 2
    for d, base in [(128, 1e6), (128, 1e4), (64, 1e4), (128, 1e6), (64, 5e5), (128, 1e4)]:
        x = torch.randn((n, H, d), generator=g)
        ref = oracle.rope(x.double().numpy(), np.arange(pos0, pos0 + n), oracle.rope_theta(d, base))
        y = jl.rope_rows(x.cuda(), pos0, rope_base=base).cpu().double().numpy()
        _say(f"[rope] d={d} base={base:g}: max err {max_abs(y, ref):.2e}")
        assert max_abs(y, ref) <= 1e-5


@pytest.mark.parametrize("dtype_name", ["bf16", "fp32"])
def test_prefill_writes_the_decode_cache(dtype_name):
    """Packed sequences with different G: the cache output of the prefill
    holds, row for row, the base-rotated keys (bitwise the row rotation at
    each sequence's positions, and the fp64 oracle's rotation within the
    dtype's rounding), and the attention outputs are bitwise those of the
    call without the cache output."""
    jl, torch = gpu_or_skip()
    dt = torch.bfloat16 if dtype_name == "bf16" else torch.float32
    Hq, Hkv, d, w0, wpt, base = (4, 2, 128, 64, 256, 1e4)
    lens = [300, 40, 1000, 513]                       # G = 2, 1, 4, 3
    cu = [0]
    for n in lens:
        cu.append(cu[-1] + n)
    T = cu[-1]
    g = torch.Generator("cpu").manual_seed(23)
    q = torch.randn((T, Hq, d), generator=g).to(dt)
    k = torch.randn((T, Hkv, d), generator=g).to(dt)
    v = torch.randn((T, Hkv, d), generator=g).to(dt)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    kc = torch.full((T, Hkv, d), float("nan"), dtype=dt, device="cuda")
    o1, l1 = jl.prefill(qd, kd, vd, w0=w0, w_pretrained=wpt, rope_base=base, cu_seqlens=cu, k_cache_out=kc)
    o0, l0 = jl.prefill(qd, kd, vd, w0=w0, w_pretrained=wpt, rope_base=base, cu_seqlens=cu)
    torch.cuda.synchronize()
    ib = torch.int16 if dt == torch.bfloat16 else torch.int32
    assert torch.equal(o1.view(ib), o0.view(ib)) and torch.equal(l1, l0)
    theta = oracle.rope_theta(d, base)
    for b, n in enumerate(lens):
        rows = kc[cu[b]:cu[b + 1]]
        ref_bits = jl.rope_rows(kd[cu[b]:cu[b + 1]], 0, rope_base=base)
        assert torch.equal(rows.view(ib), ref_bits.view(ib)), f"sequence {b}"
        ref = oracle.rope(k[cu[b]:cu[b + 1]].double().numpy(), np.arange(n), theta)
        got = rows.cpu().double().numpy()
        err = np.abs(got - ref)
        _say(f"[kcache] {dtype_name} seq {b} L={n} G={jl.group_size(n, wpt)}: max err {err.max():.2e}")
        if dt == torch.bfloat16:
            assert np.all(err <= 2.0 ** -8 * np.abs(ref) + 1e-6)   # one bf16 rounding of the rotated key
        else:
            assert err.max() <= 1e-5                               # fp32 rotation against fp64 angles
    assert not torch.isnan(kc).any()                  # every row written


def test_prefill_cache_output_rejects():
    jl, torch = gpu_or_skip()
    q = torch.zeros((64, 4, 128), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((64, 2, 128), dtype=torch.bfloat16, device="cuda")
    v = torch.zeros_like(k)
    with pytest.raises(ValueError):                    # wrong shape
        jl.prefill(q, k, v, w0=16, w_pretrained=32, rope_base=1e4, k_cache_out=torch.zeros_like(q))
    with pytest.raises(ValueError):                    # the disjoint form has no cache output
        jl.prefill(q, k, v, w0=16, w_pretrained=32, rope_base=1e4, disjoint=True, k_cache_out=torch.zeros_like(k))
    with pytest.raises(ValueError):                    # the cache output may not alias k
        jl.prefill(q, k, v, w0=16, w_pretrained=32, rope_base=1e4, k_cache_out=k)


def test_rope_rows_empty_and_rejects():
    jl, torch = gpu_or_skip()
    x = torch.zeros((0, 2, 128), dtype=torch.bfloat16, device="cuda")
    jl.rope_rows(x, 5, rope_base=1e4)                       # n = 0: nothing to do
    y = torch.zeros((4, 2, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(jl.JetLongError):
        jl.rope_rows(y, 2**31 - 2, rope_base=1e4)           # last position past 2^31 - 1
    with pytest.raises(jl.JetLongError):
        jl.rope_rows(y, -1, rope_base=1e4)


def test_streaming_chain_across_g_boundary():
    """Prefill 32766 tokens and build the base-RoPE cache from the same keys,
    then generate 5 tokens (L = 32767 .. 32771), appending each token's
    rotated key and value; G steps from 1 to 2 between L = 32768 and 32769."""
    jl, torch = gpu_or_skip()
    Hq, Hkv, d, w0, wpt, base = 32, 8, 128, 4096, 32768, 1e6
    L0, L_end = 32766, 32771
    g = torch.Generator("cpu").manual_seed(17)
    q = torch.randn((L_end, Hq, d), generator=g).to(torch.bfloat16)
    k = torch.randn((L_end, Hkv, d), generator=g).to(torch.bfloat16)
    v = torch.randn((L_end, Hkv, d), generator=g).to(torch.bfloat16)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    assert jl.group_size(32768, wpt) == 1 and jl.group_size(32769, wpt) == 2

    # prefill of the prompt, writing the cache of its base-rotated keys on the way
    cap = L_end + 3
    k_cache = torch.zeros((cap, Hkv, d), dtype=torch.bfloat16, device="cuda")
    v_cache = torch.zeros((cap, Hkv, d), dtype=torch.bfloat16, device="cuda")
    v_cache[:L0] = vd[:L0]
    o_pf, lse_pf = jl.prefill(qd[:L0], kd[:L0], vd[:L0], w0=w0, w_pretrained=wpt, rope_base=base,
                              k_cache_out=k_cache[:L0])
    # the same cache rows from the row rotation, and the same attention without the cache output
    k_rows = jl.rope_rows(kd[:L0], 0, rope_base=base)
    o_plain, lse_plain = jl.prefill(qd[:L0], kd[:L0], vd[:L0], w0=w0, w_pretrained=wpt, rope_base=base)
    torch.cuda.synchronize()
    assert torch.equal(k_cache[:L0].view(torch.int16), k_rows.view(torch.int16))
    assert torch.equal(o_pf.view(torch.int16), o_plain.view(torch.int16))
    assert torch.equal(lse_pf, lse_plain)
    assert not k_cache[L0:].any()                      # nothing written past the prompt
    prompt_k, prompt_v = k_cache[:L0].clone(), v_cache[:L0].clone()

    ws = torch.empty(jl.decode_workspace_bytes(L_end, Hq, Hkv), dtype=torch.uint8, device="cuda")
    for L in range(L0 + 1, L_end + 1):
        i = L - 1
        jl.rope_rows(kd[i:L], i, rope_base=base, out=k_cache[i:L])    # append the new token
        v_cache[i] = vd[i]
        q_i = jl.rope_rows(qd[i:L], i, rope_base=base)[0]
        o, lse = jl.decode(q_i, k_cache, v_cache, L, w0=w0, w_pretrained=wpt, rope_base=base, workspace=ws)
        o_lib, lse_lib = jl.prefill(qd[:L], kd[:L], vd[:L], w0=w0, w_pretrained=wpt, rope_base=base)
        torch.cuda.synchronize()
        oo, ll = oracle.prefill(q[:L].double().numpy(), k[:L].double().numpy(), v[:L].double().numpy(),
                                w0=w0, w_pretrained=wpt, rope_base=base, rows=[i])
        og, lg = o.float().cpu().numpy(), lse.cpu().numpy()
        e_o, e_l = max_abs(og, oo[0]), lse_rel_err(lg, ll[:, 0])
        e_lib = max_abs(og, o_lib[i].float().cpu().numpy())
        e_llib = lse_rel_err(lg, lse_lib[:, i].cpu().numpy())
        _say(f"[stream] L={L} G={jl.group_size(L, wpt)}: vs oracle max|do|={e_o:.3e} lse rel={e_l:.3e}; "
             f"vs library prefill max|do|={e_lib:.3e} lse rel={e_llib:.3e}")
        assert e_o <= BF16_O_ATOL and e_l <= BF16_LSE_RTOL
        assert e_lib <= BF16_O_ATOL and e_llib <= BF16_LSE_RTOL
    # the prompt's cache rows were never rewritten
    assert torch.equal(k_cache[:L0].view(torch.int16), prompt_k.view(torch.int16))
    assert torch.equal(v_cache[:L0].view(torch.int16), prompt_v.view(torch.int16))
    assert o_pf.shape == (L0, Hq, d)
