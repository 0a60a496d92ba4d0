"""Seeded synthetic inputs for the bifocal attention path.

This module is shared by the tests, ``bench.py`` and ``smoke()``; both the HIP
path and the oracle receive tensors made here.  It holds shapes and random
draws only: no position mapping, no rotation and no attention arithmetic.

The pages measure speed on long-context prefill of Qwen3 models and quality on
RULER / HELMET-RAG / PG-19 (Jet-Long technical summary, "Resultados
Experimentales"; English abstract).  Neither weights nor datasets are used
here: attention throughput does not depend on the values, so seeded N(0, 1)
projections at the Qwen3 attention-layer shapes stand in for them.

Recipe (every config):
  g = torch.Generator("cpu").manual_seed(seed)
  [varlen only] lengths = torch.randint(lo, hi + 1, (num_seqs,), generator=g)
  q, k, v = three torch.randn(..., dtype=float32, generator=g) draws, in that
  order; bf16 configs round them with .to(torch.bfloat16) (round to nearest
  even).  The same rounded tensors go to the GPU and, widened to float64,
  to the oracle.

Decode caches are drawn the same way: K and V caches of i.i.d. N(0, 1) values
stand for keys that were stored after base RoPE at their absolute positions.
A rotation maps an isotropic Gaussian vector to an isotropic Gaussian vector,
so a rotated N(0, 1) key and a fresh N(0, 1) draw have the same distribution.
"""

from __future__ import annotations

import dataclasses
from typing import List, Optional

import torch


@dataclasses.dataclass(frozen=True)
class PrefillConfig:
    name: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    seqlens: tuple            # one entry per packed sequence
    w0: int
    w_pretrained: int
    rope_base: float
    dtype: str                # "bf16" or "fp32"
    seed: int

    @property
    def total_tokens(self) -> int:
        return int(sum(self.seqlens))


@dataclasses.dataclass(frozen=True)
class DecodeConfig:
    name: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    L: int                    # cached keys, the current token included
    w0: int
    w_pretrained: int
    rope_base: float
    seed: int


def _varlen_lengths(seed: int, num: int, lo: int, hi: int) -> tuple:
    g = torch.Generator("cpu").manual_seed(seed)
    return tuple(int(x) for x in torch.randint(lo, hi + 1, (num,), generator=g))


# Attention-layer shapes of the Qwen3 models the pages evaluate (1.7B: 16 q /
# 8 kv heads, 4B and 8B: 32 q / 8 kv heads, head_dim 128, RoPE base 1e6,
# native window 32768).
TINY = PrefillConfig("tiny_fp32_L256", 1, 1, 64, (256,), 16, 64, 10000.0, "fp32", 0)
QWEN3_1P7B_32K = PrefillConfig("qwen3_1.7b_L32768", 16, 8, 128, (32768,), 4096, 32768, 1e6, "bf16", 1)
QWEN3_1P7B_64K = PrefillConfig("qwen3_1.7b_L65536", 16, 8, 128, (65536,), 4096, 32768, 1e6, "bf16", 1)
QWEN3_8B_128K = PrefillConfig("qwen3_8b_L131072", 32, 8, 128, (131072,), 4096, 32768, 1e6, "bf16", 2)


def varlen_4b(w0: int, seed: int = 4) -> PrefillConfig:
    """8 packed sequences, lengths uniform in [8192, 131072], Qwen3-4B heads."""
    lens = _varlen_lengths(seed, 8, 8192, 131072)
    return PrefillConfig(f"qwen3_4b_varlen8_w0{w0}", 32, 8, 128, lens, w0, 32768, 1e6, "bf16", seed)


def decode_8b(L: int, seed: int = 3) -> DecodeConfig:
    return DecodeConfig(f"qwen3_8b_decode_L{L}", 32, 8, 128, L, 4096, 32768, 1e6, seed)


DECODE_LENGTHS = (16384, 32768, 32769, 65536, 65537, 131072)


def make_prefill_inputs(cfg: PrefillConfig, seed: Optional[int] = None):
    """Returns (q, k, v) on the CPU, packed [T, H, d] in the config's dtype."""
    g = torch.Generator("cpu").manual_seed(cfg.seed if seed is None else seed)
    T = cfg.total_tokens
    q = torch.randn((T, cfg.num_q_heads, cfg.head_dim), dtype=torch.float32, generator=g)
    k = torch.randn((T, cfg.num_kv_heads, cfg.head_dim), dtype=torch.float32, generator=g)
    v = torch.randn((T, cfg.num_kv_heads, cfg.head_dim), dtype=torch.float32, generator=g)
    if cfg.dtype == "bf16":
        q, k, v = q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16)
    return q, k, v


def make_decode_inputs(cfg: DecodeConfig, L_cap: Optional[int] = None, seed: Optional[int] = None):
    """Returns (q, k_cache, v_cache) on the CPU in bf16.

    q is [Hq, d]; the caches are [L_cap, Hkv, d] with the first ``cfg.L`` rows
    valid (rows past L are drawn too, so a kernel that reads past L would see
    finite values rather than zeros)."""
    g = torch.Generator("cpu").manual_seed(cfg.seed if seed is None else seed)
    L_cap = cfg.L if L_cap is None else L_cap
    q = torch.randn((cfg.num_q_heads, cfg.head_dim), dtype=torch.float32, generator=g)
    k = torch.randn((L_cap, cfg.num_kv_heads, cfg.head_dim), dtype=torch.float32, generator=g)
    v = torch.randn((L_cap, cfg.num_kv_heads, cfg.head_dim), dtype=torch.float32, generator=g)
    return q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16)


def make_decode_batch_inputs(num_q_heads: int, num_kv_heads: int, head_dim: int, lens, seed: int,
                             gap: int = 0, device: str = "cpu"):
    """Returns (q [B, Hq, d], k_cache [R, Hkv, d], v_cache, row0) in bf16.

    Sequence b's keys occupy cache rows row0[b] .. row0[b] + lens[b] - 1; the
    sequences follow one another with ``gap`` spare rows after each (drawn
    too, so reads outside a sequence's rows would see finite values).  With
    device="cuda" the draws come from a generator on the GPU (large caches)."""
    g = torch.Generator(device).manual_seed(seed)
    row0, r = [], 0
    for n in lens:
        row0.append(r)
        r += int(n) + gap
    B = len(lens)
    q = torch.randn((B, num_q_heads, head_dim), dtype=torch.float32, generator=g, device=device)
    k = torch.randn((r, num_kv_heads, head_dim), dtype=torch.float32, generator=g, device=device)
    v = torch.randn((r, num_kv_heads, head_dim), dtype=torch.float32, generator=g, device=device)
    return q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16), row0


def cu_seqlens_of(seqlens) -> List[int]:
    out = [0]
    for n in seqlens:
        out.append(out[-1] + int(n))
    return out


def sample_rows(L: int, w0: int, G: int, n_random: int, seed: int) -> List[int]:
    """Query rows to compare at sizes where every row is too costly.

    Structural rows (first rows, both sides of the window edge, rows at the
    start and end of a group near the window edge, the last row) plus seeded
    random rows.  G is passed in by the caller; nothing here computes it."""
    rows = {0, 1, L - 1, L - 2}
    for r in (w0 - 2, w0 - 1, w0, w0 + 1, w0 + 2):
        if 0 <= r < L:
            rows.add(r)
    if G > 1:
        base = (w0 // G) * G
        for r in (base - 1, base, base + G - 1, base + G, base + 2 * G - 1):
            if 0 <= r < L:
                rows.add(r)
    g = torch.Generator("cpu").manual_seed(seed)
    if L > 0 and n_random > 0:
        for r in torch.randint(0, L, (n_random,), generator=g).tolist():
            rows.add(int(r))
    return sorted(r for r in rows if 0 <= r < L)
