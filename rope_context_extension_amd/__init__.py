"""Jet-Long dynamic bifocal RoPE attention on MI355X (gfx950).

Thin Python binding over the C ABI of ``libjetlong.so`` (include/jetlong.h):
argument marshalling only.  Every step of the attention path runs in the HIP
kernels of the library; PyTorch provides device memory and the stream.  There
is no fallback: if the library is missing or a call fails, an exception is
raised.

    o, lse = prefill(q, k, v, w0=4096, w_pretrained=32768, rope_base=1e6)
    o, lse = decode(q, k_cache, v_cache, L, w0=4096, w_pretrained=32768, rope_base=1e6)
    G = group_size(L, w_pretrained)
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

__all__ = ["group_size", "prefill", "prefill_workspace_bytes", "decode", "decode_workspace_bytes",
           "decode_batch", "decode_batch_workspace_bytes", "rope_rows",
           "lib", "JetLongError", "LIB_PATH", "BF16", "FP32"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libjetlong.so")
BF16, FP32 = 0, 1
BF16_MAX_SEQ_LEN = 8388544   # JL_BF16_MAX_SEQ_LEN: longest sequence of the bf16 prefill
_STATUS = {0: "JL_OK", -1: "JL_EINVAL", -2: "JL_EUNSUPPORTED", -3: "JL_ENOSPC", -4: "JL_EHIP"}

_lib = None


class JetLongError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{_STATUS.get(code, code)}: {msg}")
        self.code = code


def lib() -> ctypes.CDLL:
    """The loaded library (built by rope_context_extension_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run python -m rope_context_extension_amd.build")
        # torch ships its own HIP runtime under the same SONAME as the system
        # one; loading torch first makes the library bind to the runtime that
        # owns torch's device memory and streams.
        import torch  # noqa: F401
        L = ctypes.CDLL(LIB_PATH)
        c = ctypes
        L.jl_group_size.restype = c.c_int64
        L.jl_group_size.argtypes = [c.c_int64, c.c_int64]
        L.jl_last_error.restype = c.c_char_p
        L.jl_last_error.argtypes = []
        for f in (L.jl_bifocal_prefill, L.jl_bifocal_prefill_disjoint):
            f.restype = c.c_int
            f.argtypes = [
                c.c_void_p, c.c_void_p, c.c_void_p, c.c_void_p, c.c_void_p,      # q k v o lse
                c.POINTER(c.c_int64), c.c_int32, c.c_int64,                       # cu_seqlens nseq T
                c.c_int32, c.c_int32, c.POINTER(c.c_int32),                       # Hq Hkv q_to_kv
                c.c_int32, c.c_int, c.c_int64, c.c_int64, c.c_double, c.c_float,  # d dtype w0 wpt base scale
                c.c_void_p, c.POINTER(c.c_size_t), c.c_void_p]                    # ws ws_bytes stream
        L.jl_bifocal_decode.restype = c.c_int
        L.jl_bifocal_decode.argtypes = [
            c.c_void_p, c.c_void_p, c.c_void_p, c.c_int64, c.c_void_p, c.c_void_p,
            c.c_int32, c.c_int32, c.POINTER(c.c_int32), c.c_int32, c.c_int, c.c_int64, c.c_int64,
            c.c_double, c.c_float, c.c_void_p, c.POINTER(c.c_size_t), c.c_void_p]
        L.jl_bifocal_decode_batch.restype = c.c_int
        L.jl_bifocal_decode_batch.argtypes = [
            c.c_void_p, c.c_void_p, c.c_void_p, c.c_int64,                    # q k_cache v_cache cache_rows
            c.POINTER(c.c_int64), c.POINTER(c.c_int64), c.c_int32,            # row0 lens num_seqs
            c.c_void_p, c.c_void_p, c.c_int32, c.c_int32, c.POINTER(c.c_int32),  # o lse Hq Hkv q_to_kv
            c.c_int32, c.c_int, c.c_int64, c.c_int64, c.c_double, c.c_float,  # d dtype w0 wpt base scale
            c.c_void_p, c.POINTER(c.c_size_t), c.c_void_p]                    # ws ws_bytes stream
        L.jl_rope_rows.restype = c.c_int
        L.jl_rope_rows.argtypes = [c.c_void_p, c.c_void_p, c.c_int64, c.c_int32, c.c_int32, c.c_int,
                                   c.c_int64, c.c_double, c.c_void_p]
        L.jl_test_group_size_device.restype = c.c_int
        L.jl_test_group_size_device.argtypes = [c.c_void_p, c.c_int64, c.c_int64, c.c_void_p, c.c_void_p]
        L.jl_test_remote_pos_device.restype = c.c_int
        L.jl_test_remote_pos_device.argtypes = [c.c_int64, c.c_int64, c.c_int64, c.c_void_p, c.c_void_p]
        L.jl_test_rope_angles_device.restype = c.c_int
        L.jl_test_rope_angles_device.argtypes = [c.c_void_p, c.c_int64, c.c_int32, c.c_int32, c.c_double,
                                                 c.c_void_p, c.c_void_p, c.c_void_p]
        L.jl_set_profile_events.restype = c.c_int
        L.jl_set_profile_events.argtypes = [c.c_void_p, c.c_void_p, c.c_void_p]
        _lib = L
    return _lib


def _check(rc: int) -> None:
    if rc != 0:
        raise JetLongError(rc, lib().jl_last_error().decode())


def group_size(L: int, w_pretrained: int) -> int:
    """G = max(1, ceil(L / w_pretrained)), computed by the library."""
    g = lib().jl_group_size(int(L), int(w_pretrained))
    if g < 0:
        _check(int(g))
    return int(g)


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(device):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _i32_array(seq: Optional[Sequence[int]]):
    if seq is None:
        return None
    return (ctypes.c_int32 * len(seq))(*[int(x) for x in seq])


def _i64_array(seq: Optional[Sequence[int]]):
    if seq is None:
        return None
    return (ctypes.c_int64 * len(seq))(*[int(x) for x in seq])


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return FP32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _prefill_call(q, k, v, o, lse, cu, nseq, T, Hq, Hkv, kvmap, d, dt, w0, w_pt, base, scale,
                  ws, ws_bytes, stream, disjoint=False):
    fn = lib().jl_bifocal_prefill_disjoint if disjoint else lib().jl_bifocal_prefill
    return fn(q, k, v, o, lse, cu, nseq, T, Hq, Hkv, kvmap, d, dt, int(w0), int(w_pt), float(base),
              float(scale), ws, ctypes.byref(ws_bytes), stream)


def prefill_workspace_bytes(total_tokens: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                            dtype_code: int, *, w_pretrained: int, cu_seqlens=None,
                            q_to_kv=None) -> int:
    nseq = 1 if cu_seqlens is None else len(cu_seqlens) - 1
    n = ctypes.c_size_t(0)
    _check(_prefill_call(None, None, None, None, None, _i64_array(cu_seqlens), nseq, total_tokens,
                         num_q_heads, num_kv_heads, _i32_array(q_to_kv), head_dim, dtype_code, 0,
                         w_pretrained, 10000.0, 0.0, None, n, None))
    return int(n.value)


def prefill(q, k, v, *, w0: int, w_pretrained: int, rope_base: float, cu_seqlens=None,
            scale: Optional[float] = None, q_to_kv=None, out=None, lse=None, return_lse=True,
            workspace=None, disjoint: bool = False):
    """Bifocal causal prefill.  q [T, Hq, d], k/v [T, Hkv, d] raw projections
    (bf16 or fp32, CUDA, contiguous).  Returns (o [T, Hq, d], lse [Hq, T] fp32
    or None).  cu_seqlens: host list of packed sequence offsets.  disjoint:
    merge the window pass with a far-only pass instead of the three-pass
    inclusion-exclusion (bf16 only)."""
    import torch
    if not (q.is_cuda and k.is_cuda and v.is_cuda):
        raise ValueError("q, k, v must be GPU tensors")
    q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    dt = _dtype_code(q)
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share a dtype")
    nseq = 1 if cu_seqlens is None else len(cu_seqlens) - 1
    cu = _i64_array(cu_seqlens)
    kvmap = _i32_array(q_to_kv)
    o = torch.empty_like(q) if out is None else out
    if return_lse and lse is None:
        lse = torch.empty((Hq, T), dtype=torch.float32, device=q.device)
    n = ctypes.c_size_t(0)
    _check(_prefill_call(None, None, None, None, None, cu, nseq, T, Hq, Hkv, kvmap, d, dt, w0,
                         w_pretrained, rope_base, 0.0, None, n, None))
    if workspace is None or workspace.numel() < n.value:
        workspace = torch.empty(max(int(n.value), 1), dtype=torch.uint8, device=q.device)
    n = ctypes.c_size_t(workspace.numel())
    _check(_prefill_call(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse) if return_lse else None,
                         cu, nseq, T, Hq, Hkv, kvmap, d, dt, w0, w_pretrained, rope_base,
                         0.0 if scale is None else scale, _ptr(workspace), n, _stream(q.device),
                         disjoint))
    return o, (lse if return_lse else None)


def decode_workspace_bytes(L: int, num_q_heads: int, num_kv_heads: int, head_dim: int = 128,
                           q_to_kv=None) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().jl_bifocal_decode(None, None, None, int(L), None, None, num_q_heads, num_kv_heads,
                                   _i32_array(q_to_kv), head_dim, BF16, 0, 1, 10000.0, 0.0, None,
                                   ctypes.byref(n), None))
    return int(n.value)


def decode(q, k_cache, v_cache, L: int, *, w0: int, w_pretrained: int, rope_base: float,
           scale: Optional[float] = None, q_to_kv=None, out=None, lse=None, return_lse=True,
           workspace=None):
    """One generation step.  q [Hq, d] bf16 (base-rotated at L - 1); caches
    [L_cap, Hkv, d] bf16 holding base-rotated keys.  Returns (o [Hq, d], lse
    [Hq] or None)."""
    import torch
    Hq, d = q.shape
    Hkv = k_cache.shape[1]
    if k_cache.shape[0] < L or v_cache.shape[0] < L:
        raise ValueError("cache shorter than L")
    q = q.contiguous()
    if not (k_cache.is_contiguous() and v_cache.is_contiguous()):
        raise ValueError("caches must be contiguous")
    o = torch.empty_like(q) if out is None else out
    if return_lse and lse is None:
        lse = torch.empty((Hq,), dtype=torch.float32, device=q.device)
    kvmap = _i32_array(q_to_kv)
    dt = _dtype_code(q)
    n = ctypes.c_size_t(0)
    _check(lib().jl_bifocal_decode(None, None, None, int(L), None, None, Hq, Hkv, kvmap, d, dt,
                                   int(w0), int(w_pretrained), float(rope_base), 0.0, None,
                                   ctypes.byref(n), None))
    if workspace is None or workspace.numel() < n.value:
        workspace = torch.empty(max(int(n.value), 16), dtype=torch.uint8, device=q.device)
    n = ctypes.c_size_t(workspace.numel())
    _check(lib().jl_bifocal_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), int(L), _ptr(o),
                                   _ptr(lse) if return_lse else None, Hq, Hkv, kvmap, d, dt,
                                   int(w0), int(w_pretrained), float(rope_base),
                                   0.0 if scale is None else float(scale), _ptr(workspace),
                                   ctypes.byref(n), _stream(q.device)))
    return o, (lse if return_lse else None)


def _packed_rows(lens):
    r, acc = [], 0
    for n in lens:
        r.append(acc)
        acc += int(n)
    return r


def decode_batch_workspace_bytes(lens, num_q_heads: int, num_kv_heads: int, head_dim: int = 128, row0=None,
                                 q_to_kv=None, cache_rows: Optional[int] = None) -> int:
    lens = [int(n) for n in lens]
    row0 = _packed_rows(lens) if row0 is None else [int(r) for r in row0]
    rows = max([r + n for r, n in zip(row0, lens)] + [0]) if cache_rows is None else int(cache_rows)
    n = ctypes.c_size_t(0)
    _check(lib().jl_bifocal_decode_batch(None, None, None, rows, _i64_array(row0), _i64_array(lens), len(lens),
                                         None, None, num_q_heads, num_kv_heads, _i32_array(q_to_kv), head_dim,
                                         BF16, 0, 1, 10000.0, 0.0, None, ctypes.byref(n), None))
    return int(n.value)


def decode_batch(q, k_cache, v_cache, lens, *, w0: int, w_pretrained: int, rope_base: float, row0=None,
                 scale: Optional[float] = None, q_to_kv=None, out=None, lse=None, return_lse=True,
                 workspace=None):
    """One generation step for each of B ragged sequences.  q [B, Hq, d] bf16
    (q[b] base-rotated at lens[b] - 1); caches [R, Hkv, d] bf16 holding
    base-rotated keys, sequence b's keys at rows row0[b] .. row0[b] + lens[b] - 1
    (default: packed one after the other).  Returns (o [B, Hq, d], lse [B, Hq]
    or None); sequences with lens[b] == 0 leave their rows of o and lse
    unwritten."""
    import torch
    B, Hq, d = q.shape
    lens = [int(n) for n in lens]
    if len(lens) != B:
        raise ValueError("one length per query row")
    row0 = _packed_rows(lens) if row0 is None else [int(r) for r in row0]
    if not (k_cache.is_contiguous() and v_cache.is_contiguous()) or k_cache.shape != v_cache.shape:
        raise ValueError("caches must be contiguous and of one shape")
    R, Hkv = k_cache.shape[0], k_cache.shape[1]
    q = q.contiguous()
    o = torch.empty_like(q) if out is None else out
    if return_lse and lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    kvmap = _i32_array(q_to_kv)
    r0, ln = _i64_array(row0), _i64_array(lens)
    dt = _dtype_code(q)
    n = ctypes.c_size_t(0)
    _check(lib().jl_bifocal_decode_batch(None, None, None, R, r0, ln, B, None, None, Hq, Hkv, kvmap, d, dt,
                                         int(w0), int(w_pretrained), float(rope_base), 0.0, None,
                                         ctypes.byref(n), None))
    if workspace is None or workspace.numel() < n.value:
        workspace = torch.empty(max(int(n.value), 16), dtype=torch.uint8, device=q.device)
    n = ctypes.c_size_t(workspace.numel())
    _check(lib().jl_bifocal_decode_batch(_ptr(q), _ptr(k_cache), _ptr(v_cache), R, r0, ln, B, _ptr(o),
                                         _ptr(lse) if return_lse else None, Hq, Hkv, kvmap, d, dt, int(w0),
                                         int(w_pretrained), float(rope_base), 0.0 if scale is None else float(scale),
                                         _ptr(workspace), ctypes.byref(n), _stream(q.device)))
    return o, (lse if return_lse else None)


def rope_rows(x, pos0: int, *, rope_base: float, out=None):
    """Base RoPE of the rows of x [n, H, d] (bf16 or fp32) at positions pos0,
    pos0 + 1, ...; out may be x itself.  Returns out."""
    import torch
    if x.dim() != 3 or not x.is_contiguous():
        raise ValueError("x must be a contiguous [n, H, d] tensor")
    o = torch.empty_like(x) if out is None else out
    if o.shape != x.shape or o.dtype != x.dtype or not o.is_contiguous():
        raise ValueError("out must match x")
    n, H, d = x.shape
    _check(lib().jl_rope_rows(_ptr(x), _ptr(o), n, H, d, _dtype_code(x), int(pos0), float(rope_base),
                              _stream(x.device)))
    return o
