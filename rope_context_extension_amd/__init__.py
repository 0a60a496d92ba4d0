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
           "decode_batch", "decode_batch_workspace_bytes", "decode_noalloc", "rope_rows", "PreparedCall",
           "lib", "JetLongError", "LIB_PATH", "BF16", "FP32"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libjetlong.so")
BF16, FP32 = 0, 1
DECODE_SCRATCH_BYTES = 4259840  # JL_DECODE_SCRATCH_BYTES: partials the no-allocation decode holds
BF16_MAX_SEQ_LEN = 8388544   # JL_BF16_MAX_SEQ_LEN: longest sequence of the bf16 prefill
FP32_MAX_SEQ_LEN = 16777216  # JL_FP32_MAX_SEQ_LEN: longest sequence of the fp32 prefill
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
        L.jl_bifocal_prefill_kcache.restype = c.c_int
        L.jl_bifocal_prefill_kcache.argtypes = [
            c.c_void_p, c.c_void_p, c.c_void_p, c.c_void_p, c.c_void_p, c.c_void_p,  # q k v o lse k_cache
            c.POINTER(c.c_int64), c.c_int32, c.c_int64,                           # cu_seqlens nseq T
            c.c_int32, c.c_int32, c.POINTER(c.c_int32),                           # Hq Hkv q_to_kv
            c.c_int32, c.c_int, c.c_int64, c.c_int64, c.c_double, c.c_float,      # d dtype w0 wpt base scale
            c.c_void_p, c.POINTER(c.c_size_t), c.c_void_p]                        # ws ws_bytes stream
        L.jl_bifocal_decode.restype = c.c_int
        L.jl_bifocal_decode.argtypes = [
            c.c_void_p, c.c_void_p, c.c_void_p, c.c_int64, c.c_void_p, c.c_void_p,
            c.c_int32, c.c_int32, c.POINTER(c.c_int32), c.c_int32, c.c_int, c.c_int64, c.c_int64,
            c.c_double, c.c_float, c.c_void_p, c.POINTER(c.c_size_t), c.c_void_p]
        L.jl_bifocal_decode_noalloc.restype = c.c_int
        L.jl_bifocal_decode_noalloc.argtypes = [
            c.c_void_p, c.c_void_p, c.c_void_p, c.c_int64, c.c_void_p, c.c_void_p,
            c.c_int32, c.c_int32, c.POINTER(c.c_int32), c.c_int32, c.c_int, c.c_int64, c.c_int64,
            c.c_double, c.c_float, c.c_void_p]
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
        L.jl_test_device_shape.restype = c.c_int
        L.jl_test_device_shape.argtypes = [c.POINTER(c.c_int32), c.POINTER(c.c_int32)]
        L.jl_bench_mfma_peak.restype = c.c_int
        L.jl_bench_mfma_peak.argtypes = [c.c_int64, c.c_void_p, c.POINTER(c.c_int64), c.c_void_p]
        L.jl_bench_read_peak.restype = c.c_int
        L.jl_bench_read_peak.argtypes = [c.c_void_p, c.c_int64, c.c_int32, c.c_void_p, c.c_void_p]
        L.jl_test_decode_plan.restype = c.c_int
        L.jl_test_decode_plan.argtypes = [c.POINTER(c.c_int64), c.c_int32, c.c_int32, c.POINTER(c.c_int32),
                                          c.POINTER(c.c_int32)]
        L.jl_test_decode_prefix.restype = c.c_int
        L.jl_test_decode_prefix.argtypes = [c.POINTER(c.c_int64), c.c_int32, c.c_int32, c.POINTER(c.c_int32)]
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


def _need(cond: bool, msg: str, exc=ValueError) -> None:
    if not cond:
        raise exc(msg)


def _check_tensor(name: str, t, shape, dtype) -> None:
    """Structure of a tensor the C side will read or write through a raw
    pointer: exact shape, dtype and a contiguous layout.  Checked for every
    tensor before any device check and before any library call."""
    import torch
    _need(isinstance(t, torch.Tensor), f"{name} must be a torch.Tensor", TypeError)
    _need(tuple(t.shape) == tuple(shape), f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    _need(t.dtype == dtype, f"{name} has dtype {t.dtype}, expected {dtype}", TypeError)
    _need(t.is_contiguous(), f"{name} must be contiguous")


def _overlap(a, b) -> bool:
    """Whether two tensors' byte ranges intersect."""
    a0, b0 = a.data_ptr(), b.data_ptr()
    return a0 < b0 + b.numel() * b.element_size() and b0 < a0 + a.numel() * a.element_size()


def _check_devices(device, **tensors) -> None:
    """Every tensor lives on the same GPU as the first one."""
    for name, t in tensors.items():
        if t is None:
            continue
        _need(t.is_cuda, f"{name} must be a GPU tensor")
        _need(t.device == device, f"{name} is on {t.device}, expected {device}")


def _check_head_map(q_to_kv, Hq: int) -> None:
    if q_to_kv is not None:
        _need(len(q_to_kv) == Hq, f"q_to_kv has {len(q_to_kv)} entries, expected one per q head ({Hq})")


def _workspace(workspace, need: int, device):
    """The caller's workspace (uint8, contiguous, on the call's GPU) or a new one."""
    import torch
    if workspace is None:
        return torch.empty(max(int(need), 16), dtype=torch.uint8, device=device)
    _need(isinstance(workspace, torch.Tensor) and workspace.dim() == 1, "workspace must be a 1-D tensor")
    _check_tensor("workspace", workspace, (workspace.numel(),), torch.uint8)
    _check_devices(device, workspace=workspace)
    _need(workspace.numel() >= need, f"workspace has {workspace.numel()} bytes, {need} needed")
    return workspace


class PreparedCall:
    """One library call whose arguments were checked and marshalled once.

    Calling the object repeats that call on the same tensors (whose contents
    may change between calls) and the same stream, and returns the outputs.
    It is for launch-bound loops such as decode steps, where the per-call
    argument checks would take longer on the host than the step takes on the
    GPU.  The object keeps every tensor and host array of the call alive."""

    def __init__(self, fn, args, outputs, keep):
        self._fn, self._args, self.outputs, self._keep = fn, args, outputs, keep

    def __call__(self):
        rc = self._fn(*self._args)
        if rc != 0:
            _check(rc)
        return self.outputs


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return FP32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _prefill_call(q, k, v, o, lse, cu, nseq, T, Hq, Hkv, kvmap, d, dt, w0, w_pt, base, scale,
                  ws, ws_bytes, stream, disjoint=False, kc=None):
    if kc is not None:
        return lib().jl_bifocal_prefill_kcache(q, k, v, o, lse, kc, cu, nseq, T, Hq, Hkv, kvmap, d, dt, int(w0),
                                               int(w_pt), float(base), float(scale), ws, ctypes.byref(ws_bytes),
                                               stream)
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
            workspace=None, disjoint: bool = False, k_cache_out=None):
    """Bifocal causal prefill.  q [T, Hq, d], k/v [T, Hkv, d] raw projections
    (bf16 or fp32, CUDA, contiguous).  Returns (o [T, Hq, d], lse [Hq, T] fp32
    or None).  cu_seqlens: host list of packed sequence offsets.  disjoint:
    merge the window pass with a far-only pass instead of the three-pass
    inclusion-exclusion (bf16 only).  k_cache_out: a [T, Hkv, d] tensor of
    q's dtype that receives the base-rotated keys (each sequence's decode
    cache, the bits rope_rows gives at pos0 = 0); three-pass form only."""
    import torch
    _need(isinstance(q, torch.Tensor) and q.dim() == 3, "q must be a [T, Hq, d] tensor")
    dt = _dtype_code(q)
    T, Hq, d = q.shape
    _need(isinstance(k, torch.Tensor) and k.dim() == 3, "k must be a [T, Hkv, d] tensor")
    Hkv = k.shape[1]
    q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
    _check_tensor("k", k, (T, Hkv, d), q.dtype)
    _check_tensor("v", v, (T, Hkv, d), q.dtype)
    if out is not None:
        _check_tensor("out", out, (T, Hq, d), q.dtype)
    if return_lse and lse is not None:
        _check_tensor("lse", lse, (Hq, T), torch.float32)
    if k_cache_out is not None:
        _need(not disjoint, "k_cache_out is written by the three-pass form only")
        _check_tensor("k_cache_out", k_cache_out, (T, Hkv, d), q.dtype)
        for name, t in (("q", q), ("k", k), ("v", v), ("out", out), ("lse", lse if return_lse else None)):
            _need(t is None or not _overlap(k_cache_out, t), f"k_cache_out overlaps {name}")
    _check_head_map(q_to_kv, Hq)
    if cu_seqlens is not None:
        _need(len(cu_seqlens) >= 2 and int(cu_seqlens[0]) == 0 and int(cu_seqlens[-1]) == T,
              "cu_seqlens must start at 0 and end at the token count")
    _check_devices(q.device, q=q, k=k, v=v, out=out, lse=lse if return_lse else None, workspace=workspace,
                   k_cache_out=k_cache_out)
    # the plan follows the shape of the current device: make it the tensors' device
    with torch.cuda.device(q.device):
        nseq = 1 if cu_seqlens is None else len(cu_seqlens) - 1
        cu = _i64_array(cu_seqlens)
        kvmap = _i32_array(q_to_kv)
        n = ctypes.c_size_t(0)
        _check(_prefill_call(None, None, None, None, None, cu, nseq, T, Hq, Hkv, kvmap, d, dt, w0,
                             w_pretrained, rope_base, 0.0, None, n, None, disjoint))
        workspace = _workspace(workspace, int(n.value), q.device)
        o = torch.empty_like(q) if out is None else out
        if return_lse and lse is None:
            lse = torch.empty((Hq, T), dtype=torch.float32, device=q.device)
        n = ctypes.c_size_t(workspace.numel())
        _check(_prefill_call(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse) if return_lse else None,
                             cu, nseq, T, Hq, Hkv, kvmap, d, dt, w0, w_pretrained, rope_base,
                             0.0 if scale is None else scale, _ptr(workspace), n, _stream(q.device),
                             disjoint, None if k_cache_out is None else _ptr(k_cache_out)))
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
           workspace=None, prepare: bool = False):
    """One generation step.  q [Hq, d] bf16 (base-rotated at L - 1); caches
    [L_cap, Hkv, d] bf16 holding base-rotated keys.  Returns (o [Hq, d], lse
    [Hq] or None).  prepare=True launches nothing and returns a PreparedCall
    that runs this step (on the current stream) each time it is called."""
    import torch
    _need(isinstance(q, torch.Tensor) and q.dim() == 2, "q must be a [Hq, d] tensor")
    _need(isinstance(k_cache, torch.Tensor) and k_cache.dim() == 3, "k_cache must be a [L_cap, Hkv, d] tensor")
    Hq, d = q.shape
    Hkv = k_cache.shape[1]
    q = q.contiguous()
    _check_tensor("q", q, (Hq, d), torch.bfloat16)
    _check_tensor("k_cache", k_cache, (k_cache.shape[0], Hkv, d), torch.bfloat16)
    _check_tensor("v_cache", v_cache, tuple(k_cache.shape), torch.bfloat16)
    _need(0 <= int(L) <= k_cache.shape[0], f"L = {L} outside the cache's {k_cache.shape[0]} rows")
    if out is not None:
        _check_tensor("out", out, (Hq, d), torch.bfloat16)
    if return_lse and lse is not None:
        _check_tensor("lse", lse, (Hq,), torch.float32)
    _check_head_map(q_to_kv, Hq)
    _check_devices(q.device, q=q, k_cache=k_cache, v_cache=v_cache, out=out,
                   lse=lse if return_lse else None, workspace=workspace)
    # the plan follows the shape of the current device: make it the tensors' device
    with torch.cuda.device(q.device):
        kvmap = _i32_array(q_to_kv)
        dt = _dtype_code(q)
        n = ctypes.c_size_t(0)
        _check(lib().jl_bifocal_decode(None, None, None, int(L), None, None, Hq, Hkv, kvmap, d, dt,
                                       int(w0), int(w_pretrained), float(rope_base), 0.0, None,
                                       ctypes.byref(n), None))
        workspace = _workspace(workspace, int(n.value), q.device)
        o = torch.empty_like(q) if out is None else out
        if return_lse and lse is None:
            lse = torch.empty((Hq,), dtype=torch.float32, device=q.device)
        n = ctypes.c_size_t(workspace.numel())
        args = (_ptr(q), _ptr(k_cache), _ptr(v_cache), int(L), _ptr(o), _ptr(lse) if return_lse else None,
                Hq, Hkv, kvmap, d, dt, int(w0), int(w_pretrained), float(rope_base),
                0.0 if scale is None else float(scale), _ptr(workspace), ctypes.byref(n), _stream(q.device))
        outputs = (o, lse if return_lse else None)
        call = PreparedCall(lib().jl_bifocal_decode, args, outputs, (q, k_cache, v_cache, workspace, kvmap, n))
        if prepare:
            return call
        return call()


def decode_noalloc(q, k_cache, v_cache, L: int, *, w0: int, w_pretrained: int, rope_base: float,
                   scale: Optional[float] = None, q_to_kv=None, out=None, lse=None):
    """The decode step of decode() through jl_bifocal_decode_noalloc: the
    library allocates nothing and takes its partial results from its own
    device scratch (JL_DECODE_SCRATCH_BYTES per GPU).  Pass out (and lse) to
    keep the call itself free of allocation; calls that overlap in time on
    one GPU share that scratch and race.  Returns (o, lse or None)."""
    import torch
    _need(isinstance(q, torch.Tensor) and q.dim() == 2, "q must be a [Hq, d] tensor")
    _need(isinstance(k_cache, torch.Tensor) and k_cache.dim() == 3, "k_cache must be a [L_cap, Hkv, d] tensor")
    Hq, d = q.shape
    Hkv = k_cache.shape[1]
    _check_tensor("q", q, (Hq, d), torch.bfloat16)
    _check_tensor("k_cache", k_cache, (k_cache.shape[0], Hkv, d), torch.bfloat16)
    _check_tensor("v_cache", v_cache, tuple(k_cache.shape), torch.bfloat16)
    _need(0 <= int(L) <= k_cache.shape[0], f"L = {L} outside the cache's {k_cache.shape[0]} rows")
    if out is not None:
        _check_tensor("out", out, (Hq, d), torch.bfloat16)
    if lse is not None:
        _check_tensor("lse", lse, (Hq,), torch.float32)
    _check_head_map(q_to_kv, Hq)
    _check_devices(q.device, q=q, k_cache=k_cache, v_cache=v_cache, out=out, lse=lse)
    with torch.cuda.device(q.device):
        o = torch.empty_like(q) if out is None else out
        _check(lib().jl_bifocal_decode_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), int(L), _ptr(o), _ptr(lse),
                                               Hq, Hkv, _i32_array(q_to_kv), d, _dtype_code(q), int(w0),
                                               int(w_pretrained), float(rope_base),
                                               0.0 if scale is None else float(scale), _stream(q.device)))
    return o, lse


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
                 workspace=None, prepare: bool = False):
    """One generation step for each of B ragged sequences.  q [B, Hq, d] bf16
    (q[b] base-rotated at lens[b] - 1); caches [R, Hkv, d] bf16 holding
    base-rotated keys, sequence b's keys at rows row0[b] .. row0[b] + lens[b] - 1
    (default: packed one after the other).  Returns (o [B, Hq, d], lse [B, Hq]
    or None); sequences with lens[b] == 0 leave their rows of o and lse
    unwritten.  prepare=True returns a PreparedCall instead of launching."""
    import torch
    _need(isinstance(q, torch.Tensor) and q.dim() == 3, "q must be a [B, Hq, d] tensor")
    _need(isinstance(k_cache, torch.Tensor) and k_cache.dim() == 3, "k_cache must be a [R, Hkv, d] tensor")
    B, Hq, d = q.shape
    lens = [int(n) for n in lens]
    _need(len(lens) == B, f"{len(lens)} lengths for {B} query rows")
    row0 = _packed_rows(lens) if row0 is None else [int(r) for r in row0]
    _need(len(row0) == B, f"{len(row0)} first rows for {B} query rows")
    R, Hkv = k_cache.shape[0], k_cache.shape[1]
    q = q.contiguous()
    _check_tensor("q", q, (B, Hq, d), torch.bfloat16)
    _check_tensor("k_cache", k_cache, (R, Hkv, d), torch.bfloat16)
    _check_tensor("v_cache", v_cache, (R, Hkv, d), torch.bfloat16)
    if out is not None:
        _check_tensor("out", out, (B, Hq, d), torch.bfloat16)
    if return_lse and lse is not None:
        _check_tensor("lse", lse, (B, Hq), torch.float32)
    _check_head_map(q_to_kv, Hq)
    _check_devices(q.device, q=q, k_cache=k_cache, v_cache=v_cache, out=out,
                   lse=lse if return_lse else None, workspace=workspace)
    # the plan follows the shape of the current device: make it the tensors' device
    with torch.cuda.device(q.device):
        kvmap = _i32_array(q_to_kv)
        r0, ln = _i64_array(row0), _i64_array(lens)
        dt = _dtype_code(q)
        n = ctypes.c_size_t(0)
        _check(lib().jl_bifocal_decode_batch(None, None, None, R, r0, ln, B, None, None, Hq, Hkv, kvmap, d, dt,
                                             int(w0), int(w_pretrained), float(rope_base), 0.0, None,
                                             ctypes.byref(n), None))
        workspace = _workspace(workspace, int(n.value), q.device)
        o = torch.empty_like(q) if out is None else out
        if return_lse and lse is None:
            lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
        n = ctypes.c_size_t(workspace.numel())
        args = (_ptr(q), _ptr(k_cache), _ptr(v_cache), R, r0, ln, B, _ptr(o), _ptr(lse) if return_lse else None,
                Hq, Hkv, kvmap, d, dt, int(w0), int(w_pretrained), float(rope_base),
                0.0 if scale is None else float(scale), _ptr(workspace), ctypes.byref(n), _stream(q.device))
        outputs = (o, lse if return_lse else None)
        call = PreparedCall(lib().jl_bifocal_decode_batch, args, outputs,
                            (q, k_cache, v_cache, workspace, kvmap, r0, ln, n))
        if prepare:
            return call
        return call()


def rope_rows(x, pos0: int, *, rope_base: float, out=None):
    """Base RoPE of the rows of x [n, H, d] (bf16 or fp32) at positions pos0,
    pos0 + 1, ...; out may be x itself.  Returns out."""
    import torch
    _need(isinstance(x, torch.Tensor) and x.dim() == 3, "x must be an [n, H, d] tensor")
    _check_tensor("x", x, tuple(x.shape), x.dtype)
    dt = _dtype_code(x)
    if out is not None:
        _check_tensor("out", out, tuple(x.shape), x.dtype)
    _check_devices(x.device, x=x, out=out)
    o = torch.empty_like(x) if out is None else out
    n, H, d = x.shape
    _check(lib().jl_rope_rows(_ptr(x), _ptr(o), n, H, d, dt, int(pos0), float(rope_base),
                              _stream(x.device)))
    return o
