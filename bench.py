"""Benchmark of the bifocal attention hot path on one MI355X.

One step = one bifocal prefill of a Qwen3-8B-shaped attention layer (32 q / 8
kv heads, head_dim 128, bf16, RoPE base 1e6, w_pretrained 32768, w0 4096) at
L = 131072 (G = 4), followed by one single-batch decode step against a bf16
base-RoPE KV cache of L = 131072 keys.  Decode rotates through 2 GiB of
distinct cache rows, so the 256 MB last-level cache cannot hold the rows a
step reads.

Prints ONE JSON line:
  value     prefill throughput on the three-pass FLOP basis,
            F_3pass = 4 d Hq (L(L+1)/2 + 2 W), W = sum_i min(i+1, w0),
            over the whole prefill call (RoPE pre-pass included, inputs
            resident in HBM), timed with HIP events on the stream;
  roofline  the dominant kernel: the three-pass kernel of rows >= 128 (pass 1,
            then passes 3 and 2 from one walk over the remote-grid tiles,
            and the merge) with the pass-2 kernel of the first 128 rows;
            its algorithmic FLOPs on the method's three-pass basis (as
            value: 4 d Hq (L(L+1)/2 + 2 W) less passes 1 and 3 of the first
            128 rows, which run after it), over its own duration, taken
            from events the library records right around it, against the
            MI355X dense bf16 MFMA peak (and against the measured MFMA-only
            ceiling); traffic comes from the committed counter summary when it
            was measured on the current kernel source;
  decode    sustained decode steps at 128K (KV bytes 2 L Hkv d 2 per step; both
            kernels of a step, timed over back-to-back steps: the median of 3
            batches after about 30 ms of warm-up steps, since a batch timed
            from idle runs before the clocks have ramped up) against the HBM
            peak; decode_lengths: the same at 16K, 32K, 32769, 64K, 65537 and
            128K keys, bifocal and Delta-free (plain) side by side;
  prefill_configs  the other prefill workloads: Qwen3-1.7B heads at 32K (G=1)
            and 64K (G=2), and the Qwen3-4B varlen layer (8 sequences of
            8K..128K) at w0 = 1024, 4096, 8192, each on both FLOP bases (the
            median of 10 single calls after at least 3 and about 30 ms of
            warm-up calls);
  ceilings  what the chip achieves on its own: dense bf16 MFMA issue only, and
            a streaming read (default and non-temporal cache policy);
  disjoint_merge  the same prefill with the far pairs computed directly (a
            window pass on the base grid plus a far-only pass on the remote
            grid, merged with two positive weights): exactly the causal pair
            count, so its actual FLOPs are 4 d Hq L(L+1)/2;
  decode_batch  one decode step for each of 8 ragged sequences (the Qwen3-4B
            varlen lengths, 8K .. 128K) in one call, KV bytes over time;
  overhead  the bifocal calls over plain attention at the same shapes (the same
            library with w_pretrained = L, i.e. G = 1: plain causal RoPE prefill
            and Delta-free decode); also the prefill call that writes the decode
            cache of its keys, beside the separate row rotation it replaces;
  cpu_baseline  the fp64 oracle on the host cores: a sample of query rows of
            the same layer (the value), the whole tiny fp32 config and whole
            decode steps (median of 3), and the full layer extrapolated from
            the sample (labelled as such).

    python bench.py [--gpus 1] [--steps 5] [--warmup 2] [--no-cpu-baseline] [--headline-only]
    python bench.py --mfma-peak | --read-peak | --copy-calibration

--headline-only skips every run but the headline prefill and decode, so that in a profiler run every
dispatch of a kernel has the headline shape.
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import platform
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "bifocal prefill TFLOP/s (% MFMA peak) + decode KV GB/s at 128K, Qwen3-8B heads"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
CSRC = os.path.join(ROOT, "rope_context_extension_amd", "csrc")
PASS2_TRAFFIC = (os.path.join(ROOT, "profiles", "prefill_pass2_traffic_qwen3_8b_L131072.txt"),
                 os.path.join(CSRC, "jl_prefill_mfma.hip"))
DECODE_TRAFFIC = (os.path.join(ROOT, "profiles", "decode_split_traffic_qwen3_8b_L131072.txt"),
                  os.path.join(CSRC, "jl_decode.hip"))
CACHE_POOL_ROWS = 131072      # rows of each of the 4 decode cache pools (4 x 2 x 256 MiB = 2 GiB)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def window_pairs(L: int, w0: int) -> int:
    """W(L, w0) = sum_{i<L} min(i+1, w0)."""
    return w0 * L - w0 * (w0 - 1) // 2 if L >= w0 else L * (L + 1) // 2


def far_flops(L: int, Hq: int, d: int, w0: int, first_rows: int = 128):
    """FLOPs of the far-only pass over rows >= first_rows: 4 d Hq sum_i max(0, i + 1 - w0)."""
    n = max(0, L - max(w0, first_rows))              # rows with far keys beyond first_rows
    hi = L - w0                                      # far count of the last row
    lo = hi - n + 1
    return 4 * d * Hq * (n * (lo + hi) // 2) if n > 0 else 0


def prefill_flops(L: int, Hq: int, d: int, w0: int):
    """(F_3pass, F_causal): FLOPs of the three passes and of causal attention."""
    P = L * (L + 1) // 2                                   # causal pairs
    return 4 * d * Hq * (P + 2 * window_pairs(L, w0)), 4 * d * Hq * P


def prefill_flops_varlen(lens, Hq: int, d: int, w0: int):
    f3 = fc = 0
    for L in lens:
        a, b = prefill_flops(int(L), Hq, d, w0)
        f3 += a
        fc += b
    return f3, fc


class HipEvents:
    """hipEvent_t handles through the HIP runtime that torch already loaded."""

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

    def record(self, e, stream):
        rc = self.hip.hipEventRecord(e, ctypes.c_void_p(stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed: {rc}")

    def elapsed_ms(self, a, b):
        self.hip.hipEventSynchronize(b)
        t = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(t), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: {rc}")
        return float(t.value)


def read_traffic(which):
    """HBM bytes per launch of a kernel from its committed counter summary
    (FETCH_SIZE + WRITE_SIZE scaled by a plain copy's reading), or None when
    the summary is missing or was taken on other kernel source."""
    summary, source = which
    if not os.path.exists(summary):
        return None
    fields = {}
    for line in open(summary):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    src_hash = hashlib.sha256(open(source, "rb").read()).hexdigest()
    if fields.get("kernel_source_sha256") != src_hash:
        return None
    try:
        return int(float(fields["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def blas_threads() -> int:
    """Threads of numpy's BLAS, which runs the oracle's products (the process's other pools, torch's
    OpenMP pool among them, do no oracle work)."""
    import numpy  # noqa: F401  (loads the BLAS whose pool is counted)
    try:
        import threadpoolctl
        n = [p.get("num_threads", 0) for p in threadpoolctl.threadpool_info()
             if p.get("user_api") == "blas" and "numpy" in p.get("filepath", "")]
        return max(n) if n else os.cpu_count()
    except Exception:
        return os.cpu_count()


def cpu_baseline(cfg, n_rows: int, seed: int = 1234):
    """The fp64 oracle on the host cores.

    value: n_rows random query rows (all heads) of the prefill layer, on the
    same F_3pass-per-row basis as the GPU value; beside it the whole tiny fp32
    config and whole decode steps (median of 3 each), and the full layer's
    time extrapolated from the sampled rate."""
    import torch
    import oracle
    import workloads as W
    threads = blas_threads()
    L = cfg.seqlens[0]
    d, Hq = cfg.head_dim, cfg.num_q_heads
    q, k, v = W.make_prefill_inputs(cfg)
    g = torch.Generator("cpu").manual_seed(seed)
    rows = sorted(set(torch.randint(L // 2, L, (n_rows,), generator=g).tolist()))
    qn = np.zeros((L,) + tuple(q.shape[1:]))
    qn[rows] = q[torch.tensor(rows)].double().numpy()
    kn = k.double().numpy()
    vn = v.double().numpy()
    del q, k, v
    t0 = time.perf_counter()
    oracle.prefill(qn, kn, vn, w0=cfg.w0, w_pretrained=cfg.w_pretrained, rope_base=cfg.rope_base, rows=rows)
    dt = time.perf_counter() - t0
    del qn, kn, vn
    flops = sum(4 * d * Hq * ((i + 1) + 2 * min(i + 1, cfg.w0)) for i in rows)
    rate = flops / dt
    F3, _ = prefill_flops(L, Hq, d, cfg.w0)

    # the tiny fp32 config, whole (every row), median of 3
    tq, tk, tv = (t.double().numpy() for t in W.make_prefill_inputs(W.TINY))
    tiny_s = []
    for _ in range(3):
        t0 = time.perf_counter()
        oracle.prefill(tq, tk, tv, w0=W.TINY.w0, w_pretrained=W.TINY.w_pretrained, rope_base=W.TINY.rope_base)
        tiny_s.append(time.perf_counter() - t0)
    tiny_F3, _ = prefill_flops(W.TINY.seqlens[0], W.TINY.num_q_heads, W.TINY.head_dim, W.TINY.w0)

    # whole decode steps (one query row against every cached key), median of 3
    dec = {}
    for Ld in (16384, 131072):
        dcfg = W.decode_8b(Ld)
        dq, dk, dv = W.make_decode_inputs(dcfg)
        dq, dk, dv = dq.double().numpy(), dk.double().numpy(), dv.double().numpy()
        ts = []
        for _ in range(3):
            t0 = time.perf_counter()
            oracle.decode(dq, dk, dv, Ld, w0=dcfg.w0, w_pretrained=dcfg.w_pretrained, rope_base=dcfg.rope_base)
            ts.append(time.perf_counter() - t0)
        s = statistics.median(ts)
        dec[str(Ld)] = {"s_per_step": round(s, 4), "kv_GB/s": round(2 * Ld * 8 * 128 * 2 / s / 1e9, 3)}
        del dq, dk, dv
    return {"value": round(rate / 1e12, 5), "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "cpu_model": cpu_model(), "os_cpu_count": os.cpu_count(),
            "sample": f"{len(rows)} random query rows in [L/2, L) x {Hq} heads of the L={L} layer "
                      f"(keys rotated up to the last sampled row), {dt:.1f} s, F_3pass-per-row basis",
            "sample_rows_x_heads_per_s": round(len(rows) * Hq / dt, 2),
            "full_layer_s_extrapolated": round(F3 / rate, 1),
            "tiny_fp32_config_full": {"s_median_of_3": round(statistics.median(tiny_s), 5),
                                      "tflops_3pass": round(tiny_F3 / statistics.median(tiny_s) / 1e12, 6)},
            "decode_full_median_of_3": dec}


def measure_ceilings(jl, torch, dev, ev, stream):
    """MFMA-only issue rate and streaming-read bandwidth on this GPU."""
    lib = jl.lib()
    sink = torch.zeros(4, dtype=torch.float32, device=dev)
    flops = ctypes.c_int64()
    out = {}
    iters = 20000
    for _ in range(2):   # warm: the clock ramps on the first launch
        jl._check(lib.jl_bench_mfma_peak(iters, ctypes.c_void_p(sink.data_ptr()), ctypes.byref(flops),
                                         ctypes.c_void_p(stream)))
    a, b = ev.create(), ev.create()
    ev.record(a, stream)
    jl._check(lib.jl_bench_mfma_peak(iters, ctypes.c_void_p(sink.data_ptr()), ctypes.byref(flops),
                                     ctypes.c_void_p(stream)))
    ev.record(b, stream)
    ms = ev.elapsed_ms(a, b)
    out["mfma_bf16_tflops"] = round(flops.value / (ms * 1e-3) / 1e12, 1)
    nbytes = 4 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    buf.fill_(1)
    for nt, key in ((0, "read_GB/s"), (1, "read_nt_GB/s")):
        for _ in range(2):
            jl._check(lib.jl_bench_read_peak(ctypes.c_void_p(buf.data_ptr()), nbytes, nt,
                                             ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(stream)))
        ts = []
        for _ in range(5):
            ev.record(a, stream)
            jl._check(lib.jl_bench_read_peak(ctypes.c_void_p(buf.data_ptr()), nbytes, nt,
                                             ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(stream)))
            ev.record(b, stream)
            ts.append(ev.elapsed_ms(a, b))
        out[key] = round(nbytes / (statistics.median(ts) * 1e-3) / 1e9, 1)
    del buf
    torch.cuda.synchronize()
    out["method"] = ("mfma: one 8-wave workgroup per CU, four independent v_mfma_f32_32x32x16_bf16 chains per "
                     f"wave, {iters} x 32 MFMAs per wave; read: 4 GiB streamed, one workgroup per CU over its "
                     "own contiguous share, eight 16-byte loads in flight per thread, median of 5")
    return out


def time_calls(ev, stream, fn, n, warm=2):
    """Mean ms per call of fn() over n back-to-back calls (events around the batch)."""
    for _ in range(warm):
        fn()
    a, b = ev.create(), ev.create()
    ev.record(a, stream)
    for _ in range(n):
        fn()
    ev.record(b, stream)
    return ev.elapsed_ms(a, b) / n


def time_steady(ev, stream, fn, n, reps=3, warm_ms=30.0):
    """Median ms per call over `reps` batches of n back-to-back calls, after
    about warm_ms of back-to-back warm-up calls.  The GPU clocks ramp up under
    load: a batch of a few ms timed from idle reads 2-6% slow (decode steps
    at 32K and 128K keys), and a decode loop in service runs at the ramped
    clocks."""
    probe = time_calls(ev, stream, fn, 8, warm=2)
    for _ in range(int(warm_ms / max(probe, 1e-3))):
        fn()
    return float(statistics.median([time_calls(ev, stream, fn, n, warm=0) for _ in range(reps)]))


def time_median(ev, stream, fn, n=10, warm=3, warm_ms=30.0):
    """Median ms of n single calls of fn(), each between its own pair of events,
    issued back to back after at least `warm` calls and about warm_ms of
    warm-up.  A prefill call of a few ms timed from idle runs before the clocks
    have ramped (the 32K prefill read 3.48-3.96 ms in one trace of four calls)."""
    a, b = ev.create(), ev.create()
    ev.record(a, stream)
    fn()
    ev.record(b, stream)
    probe = ev.elapsed_ms(a, b)
    for _ in range(max(warm - 1, int(warm_ms / max(probe, 1e-3)))):
        fn()
    es = [ev.create() for _ in range(n + 1)]
    ev.record(es[0], stream)
    for i in range(n):
        fn()
        ev.record(es[i + 1], stream)
    return float(statistics.median([ev.elapsed_ms(es[i], es[i + 1]) for i in range(n)]))


def decode_length_timings(jl, torch, W, dev, ev, stream, lengths=None, plain=True, caches=None):
    """Decode steps (32 q / 8 kv heads, d = 128, w0 = 4096, w_pretrained = 32768) at each length over
    2 GiB of distinct cache windows: bifocal and, with plain, Delta-free (w_pretrained = L: G = 1).

    caches = (pools, q, out, lse, workspace) reuses the headline run's cache pools, allocated when the
    run starts, as a server allocates its KV cache."""
    lengths = W.DECODE_LENGTHS if lengths is None else lengths
    dcfg = W.decode_8b(CACHE_POOL_ROWS)
    Hq, Hkv, d = dcfg.num_q_heads, dcfg.num_kv_heads, dcfg.head_dim
    if caches is None:
        gen = torch.Generator(device=dev).manual_seed(dcfg.seed + 1)
        pools = [(torch.randn((CACHE_POOL_ROWS, Hkv, d), generator=gen, device=dev).bfloat16(),
                  torch.randn((CACHE_POOL_ROWS, Hkv, d), generator=gen, device=dev).bfloat16()) for _ in range(4)]
        qd = torch.randn((Hq, d), generator=gen, device=dev).bfloat16()
        od = torch.empty_like(qd)
        lsed = torch.empty((Hq,), dtype=torch.float32, device=dev)
        wsd = torch.empty(max(16, jl.decode_workspace_bytes(CACHE_POOL_ROWS, Hq, Hkv)), dtype=torch.uint8,
                          device=dev)
    else:
        pools, qd, od, lsed, wsd = caches
    outd = {}
    for Lx in lengths:
        if not 1 <= Lx <= CACHE_POOL_ROWS:
            raise SystemExit(f"decode length {Lx} outside 1 .. {CACHE_POOL_ROWS}")
        row = {}
        for key, wpt in (("bifocal", dcfg.w_pretrained), ("plain", Lx)):
            if key == "plain" and not plain:
                continue
            calls = [jl.decode(qd, kc[w * Lx:(w + 1) * Lx], vc[w * Lx:(w + 1) * Lx], Lx, w0=dcfg.w0,
                               w_pretrained=wpt, rope_base=dcfg.rope_base, out=od, lse=lsed, workspace=wsd,
                               prepare=True)
                     for kc, vc in pools for w in range(CACHE_POOL_ROWS // Lx)]
            n = max(100, len(calls) * 4)
            us = 1e3 * time_steady(ev, stream, lambda it=iter(range(10**9)): calls[next(it) % len(calls)](), n)
            b = 2 * Lx * Hkv * d * 2
            row[key] = {"us_per_step": round(us, 2), "GB/s": round(b / (us * 1e-6) / 1e9, 1),
                        "frac_hbm": round(b / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}
        row["G"] = jl.group_size(Lx, dcfg.w_pretrained)
        row["kv_bytes"] = 2 * Lx * Hkv * d * 2
        if plain:
            row["bifocal_over_plain"] = round(row["bifocal"]["us_per_step"] / row["plain"]["us_per_step"], 4)
        outd[str(Lx)] = row
        log(f"[bench] decode L={Lx}: {row['bifocal']['us_per_step']} us ({row['bifocal']['frac_hbm']:.3f} of peak)"
            + (f", plain {row['plain']['us_per_step']} us" if plain else ""))
    del pools
    torch.cuda.synchronize()
    if caches is None:
        torch.cuda.empty_cache()
    return outd


PREFILL_CONFIG_NAMES = ("qwen3_1.7b_L32768", "qwen3_1.7b_L65536", "qwen3_4b_varlen8_w01024",
                        "qwen3_4b_varlen8_w04096", "qwen3_4b_varlen8_w08192")


def prefill_config_timings(jl, torch, W, dev, ev, stream, names=PREFILL_CONFIG_NAMES, calls=10):
    """Prefill throughput of the other prefill workloads: Qwen3-1.7B heads at 32K (G=1) and 64K (G=2),
    the Qwen3-4B varlen layer at w0 = 1024, 4096, 8192.  Inputs are drawn on the GPU (the timing does
    not depend on the values).  Each figure is the median of `calls` single calls after at least three
    warm-up calls and about 30 ms of warm-up."""
    known = {c.name: c for c in [W.QWEN3_1P7B_32K, W.QWEN3_1P7B_64K] + [W.varlen_4b(w) for w in (1024, 4096, 8192)]}
    res = {}
    for name in names:
        if name not in known:
            raise SystemExit(f"unknown prefill config {name!r}; known: {', '.join(known)}")
        c = known[name]
        T = c.total_tokens
        g2 = torch.Generator(device=dev).manual_seed(c.seed)
        qx = torch.randn((T, c.num_q_heads, c.head_dim), generator=g2, device=dev).bfloat16()
        kx = torch.randn((T, c.num_kv_heads, c.head_dim), generator=g2, device=dev).bfloat16()
        vx = torch.randn((T, c.num_kv_heads, c.head_dim), generator=g2, device=dev).bfloat16()
        cu = W.cu_seqlens_of(c.seqlens) if len(c.seqlens) > 1 else None
        ox = torch.empty_like(qx)
        lx = torch.empty((c.num_q_heads, T), dtype=torch.float32, device=dev)
        wsx = torch.empty(jl.prefill_workspace_bytes(T, c.num_q_heads, c.num_kv_heads, c.head_dim, jl.BF16,
                                                     w_pretrained=c.w_pretrained, cu_seqlens=cu),
                          dtype=torch.uint8, device=dev)

        def call():
            jl.prefill(qx, kx, vx, w0=c.w0, w_pretrained=c.w_pretrained, rope_base=c.rope_base, cu_seqlens=cu,
                       out=ox, lse=lx, workspace=wsx)

        ms = time_median(ev, stream, call, calls)
        f3, fc = prefill_flops_varlen(c.seqlens, c.num_q_heads, c.head_dim, c.w0)
        gs = [jl.group_size(n, c.w_pretrained) for n in c.seqlens]
        res[c.name] = {"call_ms": round(ms, 3), "tflops_3pass": round(f3 / (ms * 1e-3) / 1e12, 2),
                       "frac_3pass": round(f3 / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                       "tflops_causal_basis": round(fc / (ms * 1e-3) / 1e12, 2),
                       "frac_causal": round(fc / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                       "flops_3pass": f3, "flops_causal": fc, "w0": c.w0, "G": gs,
                       "seqlens": list(c.seqlens)}
        log(f"[bench] prefill {c.name}: {ms:.2f} ms, {res[c.name]['tflops_3pass']} TFLOP/s (F_3pass), "
            f"{res[c.name]['tflops_causal_basis']} (causal)")
        del qx, kx, vx, ox, lx, wsx
        torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=420)
    ap.add_argument("--decode-steps", type=int, default=200)
    ap.add_argument("--headline-only", action="store_true",
                    help="run the headline prefill and decode only (profiling runs: every dispatch of a kernel "
                         "then has the headline shape)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only copy a 1 GiB buffer three times (counter calibration run)")
    ap.add_argument("--mfma-peak", action="store_true", help="only measure the MFMA-only ceiling")
    ap.add_argument("--read-peak", action="store_true", help="only measure the streaming-read ceiling")
    ap.add_argument("--prefill-config", action="append", default=[], metavar="NAME",
                    help=f"only time the named prefill workload(s) ({', '.join(PREFILL_CONFIG_NAMES)}); "
                         "for per-workload profiler runs")
    ap.add_argument("--decode-length", action="append", type=int, default=[], metavar="L",
                    help="only time decode steps at these cache lengths (bifocal); for per-length profiler runs")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}): the path shards by "
              f"kv head or by sequence with no exchange, so the one-GPU figure is the per-GPU figure.",
              file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        import torch
        src = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": src.numel(), "copies": 3}), flush=True)
        return

    import torch
    import rope_context_extension_amd as jl
    import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    ev = HipEvents()
    stream = torch.cuda.current_stream(dev).cuda_stream
    lib = jl.lib()
    if args.mfma_peak or args.read_peak:
        c = measure_ceilings(jl, torch, dev, ev, stream)
        c["device"] = torch.cuda.get_device_properties(dev).name
        print(json.dumps(c), flush=True)
        return
    if args.prefill_config:
        print(json.dumps(prefill_config_timings(jl, torch, W, dev, ev, stream, names=args.prefill_config)), flush=True)
        return
    if args.decode_length:
        print(json.dumps(decode_length_timings(jl, torch, W, dev, ev, stream, args.decode_length, plain=False)),
              flush=True)
        return

    cfg = W.QWEN3_8B_128K
    L, Hq, Hkv, d = cfg.seqlens[0], cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim
    F3, Fc = prefill_flops(L, Hq, d, cfg.w0)
    log(f"[bench] inputs: {cfg.name}")
    q, k, v = (t.to(dev) for t in W.make_prefill_inputs(cfg))
    o = torch.empty_like(q)
    lse = torch.empty((Hq, L), dtype=torch.float32, device=dev)
    ws = torch.empty(jl.prefill_workspace_bytes(L, Hq, Hkv, d, jl.BF16, w_pretrained=cfg.w_pretrained),
                     dtype=torch.uint8, device=dev)

    # decode cache pools: 4 x (K, V) of 131072 rows, 2 GiB in all; a step of L keys reads one
    # L-row window of one pool, and consecutive steps take distinct windows
    dcfg = W.decode_8b(L)
    gen = torch.Generator(device=dev).manual_seed(dcfg.seed)
    pools = []
    for _ in range(4):
        kc = torch.randn((CACHE_POOL_ROWS, Hkv, d), generator=gen, device=dev).bfloat16()
        vc = torch.randn((CACHE_POOL_ROWS, Hkv, d), generator=gen, device=dev).bfloat16()
        pools.append((kc, vc))
    qd = torch.randn((Hq, d), generator=gen, device=dev).bfloat16()
    od = torch.empty_like(qd)
    lsed = torch.empty((Hq,), dtype=torch.float32, device=dev)
    wsd = torch.empty(max(16, jl.decode_workspace_bytes(CACHE_POOL_ROWS, Hq, Hkv)), dtype=torch.uint8, device=dev)

    def decode_steps(Lx: int, wpt: int):
        """Prepared decode calls of Lx keys over distinct cache windows (2 GiB in all)."""
        calls = []
        per_pool = CACHE_POOL_ROWS // Lx
        for kc, vc in pools:
            for w in range(per_pool):
                calls.append(jl.decode(qd, kc[w * Lx:(w + 1) * Lx], vc[w * Lx:(w + 1) * Lx], Lx, w0=dcfg.w0,
                                       w_pretrained=wpt, rope_base=dcfg.rope_base, out=od, lse=lsed,
                                       workspace=wsd, prepare=True))
        return calls

    head_calls = decode_steps(L, dcfg.w_pretrained)
    kv_bytes = 2 * L * Hkv * d * 2

    def prefill():
        jl.prefill(q, k, v, w0=cfg.w0, w_pretrained=cfg.w_pretrained, rope_base=cfg.rope_base, out=o,
                   lse=lse, workspace=ws)

    log(f"[bench] warmup {args.warmup}")
    for i in range(args.warmup):
        prefill()
        head_calls[i % len(head_calls)]()
    torch.cuda.synchronize()

    # per step: [call start, attention start, after pass 2, attention end, call end] for
    # prefill, and [start, after split-K, end] for decode
    recs = [[ev.create() for _ in range(8)] for _ in range(args.steps)]
    log(f"[bench] timed {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        r = recs[i]
        ev.record(r[0], stream)
        lib.jl_set_profile_events(r[1], r[2], r[3])
        prefill()
        lib.jl_set_profile_events(None, None, None)
        ev.record(r[4], stream)
        lib.jl_set_profile_events(r[5], r[6], r[7])
        head_calls[i % len(head_calls)]()
        lib.jl_set_profile_events(None, None, None)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    call_ms = float(np.mean([ev.elapsed_ms(r[0], r[4]) for r in recs]))
    pass2_ms = float(np.mean([ev.elapsed_ms(r[1], r[2]) for r in recs]))
    attn_ms = float(np.mean([ev.elapsed_ms(r[1], r[3]) for r in recs]))
    dec_in_step_us = float(np.mean([ev.elapsed_ms(r[5], r[7]) for r in recs])) * 1e3

    # sustained decode: back-to-back steps over the rotated cache windows
    dec_us = 1e3 * time_steady(ev, stream, lambda it=iter(range(10**9)): head_calls[next(it) % len(head_calls)](),
                               args.decode_steps)
    torch.cuda.synchronize()

    def run_extras():
        """The disjoint-merge variant and plain attention at the same shapes, on the inputs above."""
        od_ = torch.empty_like(o)
        lsed_ = torch.empty_like(lse)

        def prefill_disjoint():
            jl.prefill(q, k, v, w0=cfg.w0, w_pretrained=cfg.w_pretrained, rope_base=cfg.rope_base, out=od_,
                       lse=lsed_, workspace=ws, disjoint=True)

        prefill_disjoint()
        torch.cuda.synchronize()
        drec = [[ev.create() for _ in range(5)] for _ in range(3)]
        for r in drec:
            ev.record(r[0], stream)
            lib.jl_set_profile_events(r[1], r[2], r[3])
            prefill_disjoint()
            lib.jl_set_profile_events(None, None, None)
            ev.record(r[4], stream)
        torch.cuda.synchronize()
        dj_ms = float(np.mean([ev.elapsed_ms(r[0], r[4]) for r in drec]))
        dj_far_ms = float(np.mean([ev.elapsed_ms(r[1], r[2]) for r in drec]))
        Ff = far_flops(L, Hq, d, cfg.w0)
        dj_do = float((od_.float() - o.float()).abs().max().item())
        del od_, lsed_

        # the prefill that also writes the decode cache of its keys, beside the separate row rotation
        # that would otherwise build that cache (one read and one write of k)
        kc_ = torch.empty_like(k)

        def prefill_kcache():
            jl.prefill(q, k, v, w0=cfg.w0, w_pretrained=cfg.w_pretrained, rope_base=cfg.rope_base, out=o,
                       lse=lse, workspace=ws, k_cache_out=kc_)

        kc_ms = time_calls(ev, stream, prefill_kcache, 3, warm=1)
        rows_ms = time_calls(ev, stream, lambda: jl.rope_rows(k, 0, rope_base=cfg.rope_base, out=kc_), 5, warm=1)
        torch.cuda.synchronize()
        del kc_

        # plain attention at the same shapes: G = 1 (w_pretrained = L) makes every aliased position the
        # absolute one, so the same library runs plain causal RoPE attention (one full-causal pass)
        def prefill_plain():
            jl.prefill(q, k, v, w0=cfg.w0, w_pretrained=L, rope_base=cfg.rope_base, out=o, lse=lse,
                       workspace=ws)

        plain_ms = time_calls(ev, stream, prefill_plain, 3, warm=1)
        plain_calls = decode_steps(L, L)
        dec_plain_us = 1e3 * time_steady(ev, stream,
                                         lambda it=iter(range(10**9)): plain_calls[next(it) % len(plain_calls)](),
                                         args.decode_steps)
        torch.cuda.synchronize()
        dj = {"call_ms": round(dj_ms, 3), "tflops_actual": round(Fc / (dj_ms * 1e-3) / 1e12, 2),
              "frac_actual": round(Fc / (dj_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
              "three_pass_over_disjoint": round(call_ms / dj_ms, 4),
              "far_pass_ms": round(dj_far_ms, 3),
              "far_pass_tflops": round(Ff / (dj_far_ms * 1e-3) / 1e12, 2),
              "far_pass_flops": Ff,
              "max_abs_diff_vs_three_pass": dj_do}
        ov = {"prefill_plain_causal_ms": round(plain_ms, 3),
              "prefill_bifocal_over_plain": round(call_ms / plain_ms, 4),
              "decode_plain_us_per_step": round(dec_plain_us, 2),
              "decode_bifocal_over_plain": round(dec_us / dec_plain_us, 4),
              "prefill_with_cache_output_ms": round(kc_ms, 3),
              "cache_by_separate_rope_rows_ms": round(rows_ms, 3)}
        log(f"[bench] plain causal prefill {plain_ms:.2f} ms, Delta-free decode {dec_plain_us:.1f} us; "
            f"disjoint merge {dj_ms:.2f} ms (far pass {dj_far_ms:.2f} ms)")
        return dj, ov

    def run_decode_batch():
        """Ragged batched decode: one step for each of the 8 sequences of the
        Qwen3-4B varlen lengths (8K .. 128K), 32 q / 8 kv heads, caches packed."""
        lens = list(W.varlen_4b(cfg.w0).seqlens)
        qb, kb_, vb, row0 = W.make_decode_batch_inputs(Hq, Hkv, d, lens, seed=dcfg.seed, device="cuda")
        ob = torch.empty_like(qb)
        lb = torch.empty((len(lens), Hq), dtype=torch.float32, device=dev)
        step = jl.decode_batch(qb, kb_, vb, lens, row0=row0, w0=dcfg.w0, w_pretrained=dcfg.w_pretrained,
                               rope_base=dcfg.rope_base, out=ob, lse=lb, prepare=True)
        us = 1e3 * time_steady(ev, stream, step, 50)
        torch.cuda.synchronize()
        kvb = 2 * sum(lens) * Hkv * d * 2
        log(f"[bench] batched decode of {len(lens)} sequences: {us:.1f} us per step ({kvb / us / 1e3:.0f} GB/s)")
        return {"lens": lens, "us_per_step": round(us, 2), "kv_bytes": kvb,
                "GB/s": round(kvb / (us * 1e-6) / 1e9, 1), "frac_hbm": round(kvb / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}

    # Every HBM-bound leg runs before any large buffer goes back to the driver: for about 20 s after
    # several GB are freed, every stream on the device runs slower (a 4 GiB read: 6.5 against 7.2 TB/s
    # after a 40 GB free, whether its buffer was allocated before or after), which looks like the
    # freed memory being cleared in the background.  The decode legs use the pools allocated at the
    # start, as a server allocates its KV cache.
    dl_obj = None if args.headline_only else decode_length_timings(jl, torch, W, dev, ev, stream,
                                                                   caches=(pools, qd, od, lsed, wsd))
    ceil = None if args.headline_only else measure_ceilings(jl, torch, dev, ev, stream)
    dj_obj, ov_obj = (None, None) if args.headline_only else run_extras()
    db_obj = None if args.headline_only else run_decode_batch()
    del q, k, v, o, ws, pools, head_calls
    torch.cuda.empty_cache()
    pc_obj = None if args.headline_only else prefill_config_timings(jl, torch, W, dev, ev, stream)

    tflops = F3 / (call_ms * 1e-3) / 1e12
    # the bracketed kernels: every pass of rows >= 128 and pass 2 of the
    # first 128 rows, on the three-pass basis; pass 3's products are pass 2's,
    # so the MFMA pipe executes fewer (F_causal plus pass 1's, beside it)
    w_hi = 4 * d * Hq * (window_pairs(L, cfg.w0) - window_pairs(128, cfg.w0))
    F_fused = Fc + 2 * w_hi
    pass2_tflops = F_fused / (pass2_ms * 1e-3) / 1e12
    dec_gbs = kv_bytes / (dec_us * 1e-6) / 1e9
    log(f"[bench] prefill call {call_ms:.2f} ms -> {tflops:.1f} TFLOP/s (F_3pass); attention kernels "
        f"{attn_ms:.2f} ms; three-pass kernel {pass2_ms:.2f} ms -> {pass2_tflops:.1f} TFLOP/s; decode {dec_us:.1f} "
        f"us/step ({dec_gbs:.0f} GB/s)")

    roof = {"bound": "mfma", "achieved": round(pass2_tflops, 2), "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s", "frac": round(pass2_tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": read_traffic(PASS2_TRAFFIC),
            "kernel": "prefill_pp_kernel<0> + prefill_pass_kernel<0, true> (rows >= 128: pass 1, then "
                      "passes 3 and 2 from one walk over the remote-grid tiles, and the merge; the second "
                      "kernel: pass 2 of the first 128 rows)",
            "flops_per_launch": F_fused, "ms_per_launch": round(pass2_ms, 3),
            "flops_basis": "three-pass (pass 3 shares pass 2's products)",
            "tflops_causal_plus_pass1_basis": round((Fc + w_hi) / (pass2_ms * 1e-3) / 1e12, 2)}
    dec_roof = {"bound": "hbm", "achieved": round(dec_gbs, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(dec_gbs / PEAK_HBM_GBS, 4),
                "traffic": read_traffic(DECODE_TRAFFIC),
                "kernel": "decode_split_kernel + decode_reduce_kernel (one step, timed "
                          "over back-to-back steps)", "us_per_launch": round(dec_us, 2)}
    if ceil:
        roof["frac_of_measured_mfma_ceiling"] = round(pass2_tflops / ceil["mfma_bf16_tflops"], 4)
        dec_roof["frac_of_measured_nt_read_ceiling"] = round(dec_gbs / ceil["read_nt_GB/s"], 4)
    out = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "Qwen3-8B-shaped attention layer: bifocal prefill at L=131072 (G=4) "
                               "+ one decode step at L=131072",
                   "q_heads": Hq, "kv_heads": Hkv, "head_dim": d, "L": L, "w0": cfg.w0,
                   "w_pretrained": cfg.w_pretrained, "rope_base": cfg.rope_base, "batch": 1},
        "roofline": roof,
        "prefill": {"call_ms": round(call_ms, 3), "attention_ms": round(attn_ms, 3),
                    "three_pass_kernel_ms": round(pass2_ms, 3), "tflops_3pass": round(tflops, 2),
                    "frac_3pass": round(tflops / PEAK_BF16_TFLOPS, 4),
                    "tflops_causal_basis": round(Fc / (call_ms * 1e-3) / 1e12, 2),
                    "frac_causal": round(Fc / (call_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                    "flops_3pass": F3, "flops_causal": Fc},
        "decode": {"us_per_step": round(dec_us, 2), "us_in_step": round(dec_in_step_us, 2),
                   "kv_bytes": kv_bytes, "GB/s": round(dec_gbs, 1), "roofline": dec_roof,
                   "step_frac_hbm": round(dec_gbs / PEAK_HBM_GBS, 4),
                   "caches": "4 pools of 131072 rows (2 GiB of K and V); each step reads its own window"},
        "decode_lengths": dl_obj,
        "prefill_configs": pc_obj,
        "ceilings": ceil,
        "disjoint_merge": dj_obj,
        "overhead": ov_obj,
        "decode_batch": db_obj,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        torch.cuda.empty_cache()
        log(f"[bench] cpu baseline ({args.cpu_rows} rows, tiny config, decode steps)")
        out["cpu_baseline"] = cpu_baseline(cfg, args.cpu_rows)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
