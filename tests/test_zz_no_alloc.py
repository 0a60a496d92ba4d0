"""The no-allocation decode entry point (jl_bifocal_decode_noalloc) against
the workspace entry point (jl_bifocal_decode) it varies: the same kernels and
split, so the outputs must agree bit for bit.  Two calls in a row share the
library's device scratch; the second is smaller, so a stale partial left by
the first would show."""

import ctypes
import sys

import pytest

import workloads as W
from jl_testutil import BF16_LSE_RTOL, BF16_O_ATOL, gpu_or_skip, lse_rel_err, max_abs

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _noalloc(jl, torch, q, kc, vc, L, cfg, o, lse):
    """Straight through the C ABI."""
    rc = jl.lib().jl_bifocal_decode_noalloc(
        ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(kc.data_ptr()), ctypes.c_void_p(vc.data_ptr()), L,
        ctypes.c_void_p(o.data_ptr()), ctypes.c_void_p(lse.data_ptr()), q.shape[0], kc.shape[1], None, 128,
        jl.BF16, cfg.w0, cfg.w_pretrained, cfg.rope_base, 0.0,
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0, jl.lib().jl_last_error()


def test_noalloc_decode_matches_workspace_decode_twice():
    jl, torch = gpu_or_skip()
    for L, seed in ((131072, 5), (20001, 6)):        # the second call is the smaller one
        cfg = W.decode_8b(L, seed=seed)
        q, kc, vc = (t.cuda() for t in W.make_decode_inputs(cfg))
        _say(f"[noalloc] L={L} G={jl.group_size(L, cfg.w_pretrained)}")
        o_ws, l_ws = jl.decode(q, kc, vc, L, w0=cfg.w0, w_pretrained=cfg.w_pretrained, rope_base=cfg.rope_base)
        o_na = torch.full_like(q, 3.0)
        l_na = torch.full((q.shape[0],), 3.0, dtype=torch.float32, device="cuda")
        before = torch.cuda.memory_allocated()
        _noalloc(jl, torch, q, kc, vc, L, cfg, o_na, l_na)
        torch.cuda.synchronize()
        assert torch.cuda.memory_allocated() == before
        e_o = max_abs(o_na.float().cpu().numpy(), o_ws.float().cpu().numpy())
        e_l = lse_rel_err(l_na.cpu().numpy(), l_ws.cpu().numpy())
        _say(f"[noalloc] L={L}: vs workspace decode max|do|={e_o:.3e} lse rel={e_l:.3e}")
        assert e_o <= BF16_O_ATOL and e_l <= BF16_LSE_RTOL
        assert torch.equal(o_na.view(torch.int16), o_ws.view(torch.int16))
        assert torch.equal(l_na, l_ws)


def test_noalloc_binding_and_limits():
    jl, torch = gpu_or_skip()
    cfg = W.decode_8b(4097, seed=7)
    q, kc, vc = (t.cuda() for t in W.make_decode_inputs(cfg))
    kw = dict(w0=cfg.w0, w_pretrained=cfg.w_pretrained, rope_base=cfg.rope_base)
    o_ws, l_ws = jl.decode(q, kc, vc, 4097, **kw)
    o, l = jl.decode_noalloc(q, kc, vc, 4097, out=torch.empty_like(q),
                             lse=torch.empty((32,), dtype=torch.float32, device="cuda"), **kw)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o_ws.view(torch.int16)) and torch.equal(l, l_ws)
    # 64 q heads at 128K keys need twice the scratch: refused before any launch
    q64 = torch.zeros((64, 128), dtype=torch.bfloat16, device="cuda")
    big = torch.zeros((131072, 8, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(jl.JetLongError, match="no-allocation scratch"):
        jl.decode_noalloc(q64, big, big, 131072, **kw)
