"""Streaming prefill -> decode chain on the device (technical summary,
Methodology item 2: the cache holds keys rotated by base RoPE at their
absolute positions; generation applies the correction rotation on the fly and
never rewrites the cache, also when the length crosses a G boundary).

The cache is built and extended with the library's base-RoPE row rotation
(`jl_rope_rows`), the decode loop appends one token per step across
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

    # prefill of the prompt, and the cache of its base-rotated keys
    cap = L_end + 3
    k_cache = torch.zeros((cap, Hkv, d), dtype=torch.bfloat16, device="cuda")
    v_cache = torch.zeros((cap, Hkv, d), dtype=torch.bfloat16, device="cuda")
    jl.rope_rows(kd[:L0], 0, rope_base=base, out=k_cache[:L0])
    v_cache[:L0] = vd[:L0]
    o_pf, _ = jl.prefill(qd[:L0], kd[:L0], vd[:L0], w0=w0, w_pretrained=wpt, rope_base=base)
    torch.cuda.synchronize()
    prompt_sum = k_cache[:L0].view(torch.int16).sum(dtype=torch.int64).item()

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
    assert k_cache[:L0].view(torch.int16).sum(dtype=torch.int64).item() == prompt_sum
    assert o_pf.shape == (L0, Hq, d)
