"""Benchmark of the bifocal attention hot path on one MI355X.

One step = one bifocal prefill of a Qwen3-8B-shaped attention layer (32 q / 8
kv heads, head_dim 128, bf16, RoPE base 1e6, w_pretrained 32768, w0 4096) at
L = 131072 (G = 4) followed by one single-batch decode step against a bf16
base-RoPE KV cache of L = 131072 keys (four caches are rotated so that the
256 MB last-level cache cannot hold the one being read).

Prints ONE JSON line.  `value` is prefill throughput on the three-pass FLOP
basis F_3pass = 4 d Hq (L(L+1)/2 + 2 W), W = sum_i min(i+1, w0), divided by
the measured prefill time.  The roofline object is for the dominant kernel
(the MFMA attention kernel, timed with HIP events recorded on its stream
immediately around its launches); decode is reported beside it against HBM
bandwidth.  cpu_baseline times the fp64 oracle on a sample of query rows of
the same layer.

    python bench.py [--gpus 1] [--steps 5] [--warmup 2] [--no-cpu-baseline]
"""

from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "bifocal prefill TFLOP/s (% MFMA peak) + decode KV GB/s at 128K, Qwen3-8B heads"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def prefill_flops(L: int, Hq: int, d: int, w0: int):
    P = L * (L + 1) // 2                                   # causal pairs
    W = w0 * L - w0 * (w0 - 1) // 2 if L >= w0 else P      # window pairs, sum_i min(i+1, w0)
    return 4 * d * Hq * (P + 2 * W), 4 * d * Hq * P


class HipEvents:
    """hipEvent_t pairs through the HIP runtime that torch already loaded."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]

    def create(self):
        e = ctypes.c_void_p()
        rc = self.hip.hipEventCreate(ctypes.byref(e))
        if rc != 0:
            raise RuntimeError(f"hipEventCreate failed: {rc}")
        return e

    def elapsed_ms(self, a, b):
        self.hip.hipEventSynchronize(b)
        t = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(t), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: {rc}")
        return float(t.value)


def cpu_baseline(cfg, n_rows: int, seed: int = 1234):
    """fp64 oracle on n_rows random query rows (all heads) of the prefill
    layer; throughput on the same F_3pass-per-row basis as the GPU value."""
    import torch
    import oracle
    import workloads as W
    try:
        import threadpoolctl
        threads = sum(p.get("num_threads", 0) for p in threadpoolctl.threadpool_info()) or os.cpu_count()
    except Exception:
        threads = os.cpu_count()
    L = cfg.seqlens[0]
    q, k, v = W.make_prefill_inputs(cfg)
    g = torch.Generator("cpu").manual_seed(seed)
    rows = sorted(set(torch.randint(L // 2, L, (n_rows,), generator=g).tolist()))
    qn = np.zeros((L,) + tuple(q.shape[1:]))
    qn[rows] = q[torch.tensor(rows)].double().numpy()
    kn = k.double().numpy()
    vn = v.double().numpy()
    t0 = time.perf_counter()
    oracle.prefill(qn, kn, vn, w0=cfg.w0, w_pretrained=cfg.w_pretrained, rope_base=cfg.rope_base,
                   rows=rows)
    dt = time.perf_counter() - t0
    d, Hq = cfg.head_dim, cfg.num_q_heads
    flops = sum(4 * d * Hq * ((i + 1) + 2 * min(i + 1, cfg.w0)) for i in rows)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{len(rows)} random query rows in [L/2, L) x {Hq} heads of the L={L} layer "
                      f"(keys rotated for all rows up to the last); {dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=24)
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the path shards by kv head "
              f"or sequence with no exchange, so one GPU's figure is the per-GPU figure.", file=sys.stderr)
        sys.exit(2)

    import torch
    import rope_context_extension_amd as jl
    import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = W.QWEN3_8B_128K
    L, Hq, Hkv, d = cfg.seqlens[0], cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim
    F3, Fc = prefill_flops(L, Hq, d, cfg.w0)
    log(f"[bench] inputs: {cfg.name}")
    q, k, v = (t.to(dev) for t in W.make_prefill_inputs(cfg))
    o = torch.empty_like(q)
    lse = torch.empty((Hq, L), dtype=torch.float32, device=dev)
    ws = torch.empty(jl.prefill_workspace_bytes(L, Hq, Hkv, d, jl.BF16, w_pretrained=cfg.w_pretrained),
                     dtype=torch.uint8, device=dev)

    dcfg = W.decode_8b(L)
    n_caches = 4
    gen = torch.Generator(device=dev).manual_seed(dcfg.seed)
    caches = []
    for _ in range(n_caches):
        kc = torch.randn((L, Hkv, d), generator=gen, device=dev).bfloat16()
        vc = torch.randn((L, Hkv, d), generator=gen, device=dev).bfloat16()
        caches.append((kc, vc))
    qd = torch.randn((Hq, d), generator=gen, device=dev).bfloat16()
    od = torch.empty_like(qd)
    lsed = torch.empty((Hq,), dtype=torch.float32, device=dev)
    wsd = torch.empty(max(16, jl.decode_workspace_bytes(L, Hq, Hkv)), dtype=torch.uint8, device=dev)
    kv_bytes = 2 * L * Hkv * d * 2

    ev = HipEvents()
    stream = torch.cuda.current_stream(dev)

    def step(i, rec=None):
        if rec is not None:
            jl.lib().jl_set_profile_events(rec[0], rec[1])
        jl.prefill(q, k, v, w0=cfg.w0, w_pretrained=cfg.w_pretrained, rope_base=cfg.rope_base, out=o,
                   lse=lse, workspace=ws)
        if rec is not None:
            jl.lib().jl_set_profile_events(rec[2], rec[3])
        kc, vc = caches[i % n_caches]
        jl.decode(qd, kc, vc, L, w0=dcfg.w0, w_pretrained=dcfg.w_pretrained, rope_base=dcfg.rope_base,
                  out=od, lse=lsed, workspace=wsd)
        if rec is not None:
            jl.lib().jl_set_profile_events(None, None)

    log(f"[bench] warmup {args.warmup}")
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    recs = [tuple(ev.create() for _ in range(4)) for _ in range(args.steps)]
    # decode alone, many back-to-back steps over the rotated caches
    n_dec = 200
    dec_ev = (ev.create(), ev.create())
    log(f"[bench] timed {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, recs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    pre_ms = [ev.elapsed_ms(r[0], r[1]) for r in recs]
    dec_ms = [ev.elapsed_ms(r[2], r[3]) for r in recs]
    jl.lib().jl_set_profile_events(None, None)

    # sustained decode: n_dec steps between two events on the stream
    torch.cuda.synchronize()
    jl.lib().jl_set_profile_events(None, None)
    ev.hip.hipEventRecord(dec_ev[0], ctypes.c_void_p(stream.cuda_stream))
    for i in range(n_dec):
        kc, vc = caches[i % n_caches]
        jl.decode(qd, kc, vc, L, w0=dcfg.w0, w_pretrained=dcfg.w_pretrained, rope_base=dcfg.rope_base,
                  out=od, lse=lsed, workspace=wsd)
    ev.hip.hipEventRecord(dec_ev[1], ctypes.c_void_p(stream.cuda_stream))
    dec_loop_us = ev.elapsed_ms(*dec_ev) * 1e3 / n_dec
    torch.cuda.synchronize()

    pre_kernel_ms = float(np.mean(pre_ms))
    dec_kernel_us = float(np.mean(dec_ms)) * 1e3
    ms_per_step = wall * 1e3 / args.steps
    tflops = F3 / (pre_kernel_ms * 1e-3) / 1e12
    dec_gbs = kv_bytes / (dec_loop_us * 1e-6) / 1e9
    log(f"[bench] prefill kernel {pre_kernel_ms:.2f} ms -> {tflops:.1f} TFLOP/s (F_3pass), "
        f"{Fc / (pre_kernel_ms * 1e-3) / 1e12:.1f} (F_causal); decode {dec_loop_us:.1f} us/step "
        f"({dec_gbs:.0f} GB/s), in-step {dec_kernel_us:.1f} us")

    out = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "Qwen3-8B attention layer: bifocal prefill L=131072 (G=4) + decode step at L=131072",
                   "q_heads": Hq, "kv_heads": Hkv, "head_dim": d, "L": L, "w0": cfg.w0,
                   "w_pretrained": cfg.w_pretrained, "rope_base": cfg.rope_base, "batch": 1},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4), "traffic": None},
        "prefill": {"kernel_ms": round(pre_kernel_ms, 3), "tflops_3pass": round(tflops, 2),
                    "tflops_causal": round(Fc / (pre_kernel_ms * 1e-3) / 1e12, 2),
                    "flops_3pass": F3, "flops_causal": Fc},
        "decode": {"us_per_step": round(dec_loop_us, 2), "us_in_step": round(dec_kernel_us, 2),
                   "kv_bytes": kv_bytes, "GB/s": round(dec_gbs, 1),
                   "roofline": {"bound": "hbm", "achieved": round(dec_gbs, 1), "peak": PEAK_HBM_GBS,
                                "unit": "GB/s", "frac": round(dec_gbs / PEAK_HBM_GBS, 4), "traffic": None}},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        del q, k, v, o, ws, caches
        torch.cuda.empty_cache()
        log(f"[bench] cpu baseline ({args.cpu_rows} rows)")
        out["cpu_baseline"] = cpu_baseline(cfg, args.cpu_rows)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
