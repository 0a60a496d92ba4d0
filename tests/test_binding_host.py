"""Host-side tests of the Python binding's argument checks (no GPU).

The binding hands raw pointers to the C ABI, and the kernels trust every
shape they are given, so each tensor is checked (shape, dtype, contiguity,
then device) before the library is called.  Each bad argument below must
raise in the binding; CPU tensors with a correct structure must fail the
device check, so no call here can reach a launch."""

import pytest
import torch

from jl_testutil import ensure_built

jl = ensure_built()
bf = torch.bfloat16


def _prefill_args(T=40, Hq=4, Hkv=2, d=128, dtype=bf):
    return (torch.zeros((T, Hq, d), dtype=dtype), torch.zeros((T, Hkv, d), dtype=dtype),
            torch.zeros((T, Hkv, d), dtype=dtype))


KW = dict(w0=8, w_pretrained=16, rope_base=1e4)


def test_prefill_good_structure_fails_on_device_only():
    q, k, v = _prefill_args()
    with pytest.raises(ValueError, match="GPU tensor"):
        jl.prefill(q, k, v, **KW)


@pytest.mark.parametrize("case,exc,msg", [
    ("k_rows", ValueError, "k has shape"),
    ("v_heads", ValueError, "v has shape"),
    ("kv_dtype", TypeError, "dtype"),
    ("out_shape", ValueError, "out has shape"),
    ("out_dtype", TypeError, "out has dtype"),
    ("out_strided", ValueError, "out must be contiguous"),
    ("lse_shape", ValueError, "lse has shape"),
    ("lse_dtype", TypeError, "lse has dtype"),
    ("head_map", ValueError, "q_to_kv has"),
    ("cu_end", ValueError, "cu_seqlens"),
    ("q_2d", ValueError, "q must be"),
    ("q_int", TypeError, "unsupported dtype"),
    ("kcache_shape", ValueError, "k_cache_out has shape"),
    ("kcache_dtype", TypeError, "k_cache_out has dtype"),
    ("kcache_alias_k", ValueError, "k_cache_out overlaps k"),
    ("kcache_disjoint", ValueError, "three-pass form only"),
    ("kcache_cpu", ValueError, "GPU tensor"),
])
def test_prefill_rejects_bad_tensors(case, exc, msg):
    T, Hq, Hkv, d = 40, 4, 2, 128
    q, k, v = _prefill_args(T, Hq, Hkv, d)
    kw = dict(KW)
    if case == "k_rows":
        k = torch.zeros((T - 1, Hkv, d), dtype=bf)
    elif case == "v_heads":
        v = torch.zeros((T, Hkv + 1, d), dtype=bf)
    elif case == "kv_dtype":
        k = k.float()
    elif case == "out_shape":
        kw["out"] = torch.zeros((T, Hq, d - 1), dtype=bf)
    elif case == "out_dtype":
        kw["out"] = torch.zeros((T, Hq, d), dtype=torch.float32)
    elif case == "out_strided":
        kw["out"] = torch.zeros((T, d, Hq), dtype=bf).transpose(1, 2)
    elif case == "lse_shape":
        kw["lse"] = torch.zeros((T, Hq), dtype=torch.float32)
    elif case == "lse_dtype":
        kw["lse"] = torch.zeros((Hq, T), dtype=bf)
    elif case == "head_map":
        kw["q_to_kv"] = [0, 1, 0]
    elif case == "cu_end":
        kw["cu_seqlens"] = [0, 10, 30]
    elif case == "q_2d":
        q = q[0]
    elif case == "q_int":
        q = torch.zeros((T, Hq, d), dtype=torch.int16)
    elif case == "kcache_shape":
        kw["k_cache_out"] = torch.zeros((T, Hq, d), dtype=bf)
    elif case == "kcache_dtype":
        kw["k_cache_out"] = torch.zeros((T, Hkv, d), dtype=torch.float32)
    elif case == "kcache_alias_k":
        kw["k_cache_out"] = k
    elif case == "kcache_disjoint":
        kw["k_cache_out"] = torch.zeros((T, Hkv, d), dtype=bf)
        kw["disjoint"] = True
    elif case == "kcache_cpu":
        kw["k_cache_out"] = torch.zeros((T, Hkv, d), dtype=bf)   # right structure: fails on the device check
    with pytest.raises(exc, match=msg):
        jl.prefill(q, k, v, **kw)


def _decode_args(L_cap=50, Hq=8, Hkv=2, d=128):
    return (torch.zeros((Hq, d), dtype=bf), torch.zeros((L_cap, Hkv, d), dtype=bf),
            torch.zeros((L_cap, Hkv, d), dtype=bf))


def test_decode_good_structure_fails_on_device_only():
    q, kc, vc = _decode_args()
    with pytest.raises(ValueError, match="GPU tensor"):
        jl.decode(q, kc, vc, 50, **KW)


@pytest.mark.parametrize("case,exc,msg", [
    ("L_past_cache", ValueError, "outside the cache"),
    ("L_negative", ValueError, "outside the cache"),
    ("q_dtype", TypeError, "q has dtype"),
    ("q_dim", ValueError, "k_cache has shape"),
    ("k_dtype", TypeError, "k_cache has dtype"),
    ("v_shape", ValueError, "v_cache has shape"),
    ("k_strided", ValueError, "k_cache must be contiguous"),
    ("out_shape", ValueError, "out has shape"),
    ("out_dtype", TypeError, "out has dtype"),
    ("lse_shape", ValueError, "lse has shape"),
    ("head_map", ValueError, "q_to_kv has"),
    ("workspace_dtype", TypeError, "workspace has dtype"),
])
def test_decode_rejects_bad_tensors(case, exc, msg):
    Hq, Hkv, d, L = 8, 2, 128, 50
    q, kc, vc = _decode_args(L, Hq, Hkv, d)
    kw = dict(KW)
    Lc = L
    if case == "L_past_cache":
        Lc = L + 1
    elif case == "L_negative":
        Lc = -1
    elif case == "q_dtype":
        q = q.float()
    elif case == "q_dim":
        q = torch.zeros((Hq, d // 2), dtype=bf)
    elif case == "k_dtype":
        kc = kc.float()
    elif case == "v_shape":
        vc = torch.zeros((L - 1, Hkv, d), dtype=bf)
    elif case == "k_strided":
        kc = torch.zeros((Hkv, L, d), dtype=bf).transpose(0, 1)
    elif case == "out_shape":
        kw["out"] = torch.zeros((Hq + 1, d), dtype=bf)
    elif case == "out_dtype":
        kw["out"] = torch.zeros((Hq, d), dtype=torch.float32)
    elif case == "lse_shape":
        kw["lse"] = torch.zeros((Hq, 1), dtype=torch.float32)
    elif case == "head_map":
        kw["q_to_kv"] = [0] * (Hq - 1)
    elif case == "workspace_dtype":
        kw["workspace"] = torch.zeros((1 << 20,), dtype=torch.float32)
    # the workspace check runs after the structural ones and after the size
    # query; with CPU tensors everything else fails at the device check first
    if case == "workspace_dtype":
        with pytest.raises(ValueError, match="GPU tensor"):
            jl.decode(q, kc, vc, Lc, **kw)
        with pytest.raises(exc, match=msg):
            jl._workspace(kw["workspace"], 16, torch.device("cpu"))
        return
    with pytest.raises(exc, match=msg):
        jl.decode(q, kc, vc, Lc, **kw)


def test_workspace_checks():
    cpu = torch.device("cpu")
    with pytest.raises(ValueError, match="1-D"):
        jl._workspace(torch.zeros((4, 4), dtype=torch.uint8), 16, cpu)
    with pytest.raises(ValueError, match="GPU tensor"):
        jl._workspace(torch.zeros((64,), dtype=torch.uint8), 16, cpu)


def test_decode_batch_rejects_bad_arguments():
    B, Hq, Hkv, d = 3, 8, 2, 128
    q = torch.zeros((B, Hq, d), dtype=bf)
    kc = torch.zeros((100, Hkv, d), dtype=bf)
    vc = torch.zeros((100, Hkv, d), dtype=bf)
    with pytest.raises(ValueError, match="3 lengths"):
        jl.decode_batch(q[:2], kc, vc, [10, 20, 30], **KW)
    with pytest.raises(ValueError, match="2 first rows for 3"):
        jl.decode_batch(q, kc, vc, [10, 20, 30], row0=[0, 10], **KW)
    with pytest.raises(ValueError, match="v_cache has shape"):
        jl.decode_batch(q, kc, vc[:99], [10, 20, 30], **KW)
    with pytest.raises(ValueError, match="out has shape"):
        jl.decode_batch(q, kc, vc, [10, 20, 30], out=torch.zeros((B, Hq), dtype=bf), **KW)
    with pytest.raises(ValueError, match="lse has shape"):
        jl.decode_batch(q, kc, vc, [10, 20, 30], lse=torch.zeros((B,), dtype=torch.float32), **KW)
    with pytest.raises(ValueError, match="GPU tensor"):
        jl.decode_batch(q, kc, vc, [10, 20, 30], **KW)


def test_rope_rows_rejects_bad_arguments():
    x = torch.zeros((10, 2, 128), dtype=bf)
    with pytest.raises(ValueError, match="out has shape"):
        jl.rope_rows(x, 0, rope_base=1e4, out=torch.zeros((9, 2, 128), dtype=bf))
    with pytest.raises(TypeError, match="out has dtype"):
        jl.rope_rows(x, 0, rope_base=1e4, out=torch.zeros((10, 2, 128), dtype=torch.float32))
    with pytest.raises(ValueError, match="x must be contiguous"):
        jl.rope_rows(torch.zeros((2, 10, 128), dtype=bf).transpose(0, 1), 0, rope_base=1e4)
    with pytest.raises(ValueError, match="GPU tensor"):
        jl.rope_rows(x, 0, rope_base=1e4)
