"""Shared helpers for the tests: library handle, tolerances, comparisons."""

import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# Parity bars.  fp32 path: max-abs 1e-5 on o.  bf16 path (bf16 inputs, bf16
# rotated operands and probabilities, fp32 accumulation): max-abs 2e-2 on o
# and |lse - lse_ref| / max(1, |lse_ref|) <= 1e-3.
FP32_O_ATOL = 1e-5
FP32_LSE_ATOL = 1e-5
BF16_O_ATOL = 2e-2
BF16_LSE_RTOL = 1e-3


def ensure_built():
    import rope_context_extension_amd as jl
    if not os.path.exists(jl.LIB_PATH):
        from rope_context_extension_amd.build import build
        build(verbose=False)
    return jl


def gpu_or_skip():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    jl = ensure_built()
    return jl, torch


def header_symbols():
    names = []
    for h in ("jetlong.h", "jetlong_testing.h"):
        text = open(os.path.join(ROOT, "include", h)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names += re.findall(r"\b(jl_\w+)\s*\(", text)
    return sorted(set(names))


def lse_rel_err(lse, ref):
    lse = np.asarray(lse, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.max(np.abs(lse - ref) / np.maximum(1.0, np.abs(ref)))) if ref.size else 0.0


def max_abs(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b))) if a.size else 0.0
