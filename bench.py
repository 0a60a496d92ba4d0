"""Benchmark of the bifocal attention hot path on one MI355X.

One step = one bifocal prefill of a Qwen3-8B-shaped attention layer (32 q / 8
kv heads, head_dim 128, bf16, RoPE base 1e6, w_pretrained 32768, w0 4096) at
L = 131072 (G = 4), followed by one single-batch decode step against a bf16
base-RoPE KV cache of L = 131072 keys.  Four decode caches (2 GiB) are
rotated so the 256 MB last-level cache cannot hold the one being read.

Prints ONE JSON line:
  value     prefill throughput on the three-pass FLOP basis,
            F_3pass = 4 d Hq (L(L+1)/2 + 2 W), W = sum_i min(i+1, w0),
            over the whole prefill call (RoPE pre-pass included, inputs
            resident in HBM), timed with HIP events on the stream;
  roofline  the dominant kernel (the full-causal pass-2 launches): its
            algorithmic FLOPs 4 d Hq L(L+1)/2 over its own duration, taken
            from events the library records right around it, against the
            MI355X dense bf16 MFMA peak; traffic comes from the committed
            counter summary when it was measured on the current kernel source;
  decode    sustained decode steps (KV bytes 2 L Hkv d 2 per step; both
            kernels of a step, timed over back-to-back steps, since a HIP
            event pair around one ~100 us kernel adds several us of its own)
            against the HBM peak;
  disjoint_merge  the same prefill with the far pairs computed directly (a
            window pass on the base grid plus a far-only pass on the remote
            grid, merged with two positive weights): exactly the causal pair
            count, so its actual FLOPs are 4 d Hq L(L+1)/2;
  decode_batch  one decode step for each of 8 ragged sequences (the Qwen3-4B
            varlen lengths, 8K .. 128K) in one call, KV bytes over time;
  overhead  the bifocal calls over plain attention at the same shapes (the same
            library with w_pretrained = L, i.e. G = 1: plain causal RoPE prefill
            and Delta-free decode);
  cpu_baseline  the fp64 oracle on a sample of query rows of the same layer.

    python bench.py [--gpus 1] [--steps 5] [--warmup 2] [--no-cpu-baseline] [--headline-only]

--headline-only skips the disjoint-merge, plain-attention, G-boundary and batched-decode runs, so
that in a profiler run every dispatch of a kernel has the headline shape.
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
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
CSRC = os.path.join(ROOT, "rope_context_extension_amd", "csrc")
PASS2_TRAFFIC = (os.path.join(ROOT, "profiles", "prefill_pass2_traffic_qwen3_8b_L131072.txt"),
                 os.path.join(CSRC, "jl_prefill_mfma.hip"))
DECODE_TRAFFIC = (os.path.join(ROOT, "profiles", "decode_split_traffic_qwen3_8b_L131072.txt"),
                  os.path.join(CSRC, "jl_decode.hip"))


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def far_flops(L: int, Hq: int, d: int, w0: int, first_rows: int = 128):
    """FLOPs of the far-only pass over rows >= first_rows: 4 d Hq sum_i max(0, i + 1 - w0)."""
    n = max(0, L - max(w0, first_rows))              # rows with far keys beyond first_rows
    hi = L - w0                                      # far count of the last row
    lo = hi - n + 1
    return 4 * d * Hq * (n * (lo + hi) // 2) if n > 0 else 0


def prefill_flops(L: int, Hq: int, d: int, w0: int):
    """(F_3pass, F_causal): FLOPs of the three passes and of causal attention."""
    P = L * (L + 1) // 2                                   # causal pairs
    W = w0 * L - w0 * (w0 - 1) // 2 if L >= w0 else P      # window pairs, sum_i min(i+1, w0)
    return 4 * d * Hq * (P + 2 * W), 4 * d * Hq * P


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


def cpu_baseline(cfg, n_rows: int, seed: int = 1234):
    """fp64 oracle on n_rows random query rows (all heads) of the prefill layer;
    throughput on the same F_3pass-per-row basis as the GPU value."""
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
    return {"value": round(flops / dt / 1e12, 5), "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{len(rows)} random query rows in [L/2, L) x {Hq} heads of the L={L} layer "
                      f"(keys rotated up to the last sampled row), {dt:.1f} s, F_3pass-per-row basis"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=420)
    ap.add_argument("--decode-steps", type=int, default=200)
    ap.add_argument("--headline-only", action="store_true",
                    help="skip the disjoint-merge, plain-attention and G-boundary runs (profiling runs: every "
                         "dispatch of a kernel then has the headline shape)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only copy a 1 GiB buffer three times (counter calibration run)")
    args = ap.parse_args()
    if args.copy_calibration:
        import torch
        src = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": src.numel(), "copies": 3}), flush=True)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}): the path shards by "
              f"kv head or by sequence with no exchange, so the one-GPU figure is the per-GPU figure.",
              file=sys.stderr)
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
    stream = torch.cuda.current_stream(dev).cuda_stream
    lib = jl.lib()

    def prefill():
        jl.prefill(q, k, v, w0=cfg.w0, w_pretrained=cfg.w_pretrained, rope_base=cfg.rope_base, out=o,
                   lse=lse, workspace=ws)

    def decode(i):
        kc, vc = caches[i % n_caches]
        jl.decode(qd, kc, vc, L, w0=dcfg.w0, w_pretrained=dcfg.w_pretrained, rope_base=dcfg.rope_base,
                  out=od, lse=lsed, workspace=wsd)

    log(f"[bench] warmup {args.warmup}")
    for i in range(args.warmup):
        prefill()
        decode(i)
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
        decode(i)
        lib.jl_set_profile_events(None, None, None)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    call_ms = float(np.mean([ev.elapsed_ms(r[0], r[4]) for r in recs]))
    pass2_ms = float(np.mean([ev.elapsed_ms(r[1], r[2]) for r in recs]))
    attn_ms = float(np.mean([ev.elapsed_ms(r[1], r[3]) for r in recs]))
    dec_in_step_us = float(np.mean([ev.elapsed_ms(r[5], r[7]) for r in recs])) * 1e3

    # sustained decode: back-to-back steps over the rotated caches
    e0, e1 = ev.create(), ev.create()
    torch.cuda.synchronize()
    ev.record(e0, stream)
    for i in range(args.decode_steps):
        decode(i)
    ev.record(e1, stream)
    dec_us = ev.elapsed_ms(e0, e1) * 1e3 / args.decode_steps
    torch.cuda.synchronize()

    def run_extras():
        """The disjoint-merge variant, plain attention at the same shapes and decode steps on both
        sides of the G boundaries, on the inputs above."""
        # the disjoint merge variant on the same inputs (own output buffers)
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

        # overhead against plain attention at the same shapes: G = 1 (w_pretrained = L) makes every
        # aliased position the absolute one, so the same library runs plain causal RoPE attention
        # (prefill: one full-causal pass) and Delta-free decode (every key on the base path)
        def prefill_plain():
            jl.prefill(q, k, v, w0=cfg.w0, w_pretrained=L, rope_base=cfg.rope_base, out=o, lse=lse,
                       workspace=ws)

        def decode_plain(i):
            kc, vc = caches[i % n_caches]
            jl.decode(qd, kc, vc, L, w0=dcfg.w0, w_pretrained=L, rope_base=dcfg.rope_base, out=od, lse=lsed,
                      workspace=wsd)

        prefill_plain()
        torch.cuda.synchronize()
        pe = [(ev.create(), ev.create()) for _ in range(3)]
        for a_, b_ in pe:
            ev.record(a_, stream)
            prefill_plain()
            ev.record(b_, stream)
        plain_ms = float(np.mean([ev.elapsed_ms(a_, b_) for a_, b_ in pe]))
        for i in range(8):
            decode_plain(i)
        torch.cuda.synchronize()
        ev.record(e0, stream)
        for i in range(args.decode_steps):
            decode_plain(i)
        ev.record(e1, stream)
        dec_plain_us = ev.elapsed_ms(e0, e1) * 1e3 / args.decode_steps
        torch.cuda.synchronize()

        # decode step time on both sides of the G boundaries (the cache is the same; only L moves),
        # bifocal and plain (w_pretrained = L: G = 1) at each length
        def decode_at(Lx, i, wpt):
            kc, vc = caches[i % n_caches]
            jl.decode(qd, kc, vc, Lx, w0=dcfg.w0, w_pretrained=wpt, rope_base=dcfg.rope_base,
                      out=od, lse=lsed, workspace=wsd)

        boundary, boundary_plain = {}, {}
        for Lx in (32768, 32769, 65536, 65537):
            for key, wpt in ((boundary, dcfg.w_pretrained), (boundary_plain, Lx)):
                for i in range(4):
                    decode_at(Lx, i, wpt)
                torch.cuda.synchronize()
                ev.record(e0, stream)
                for i in range(100):
                    decode_at(Lx, i, wpt)
                ev.record(e1, stream)
                key[str(Lx)] = round(ev.elapsed_ms(e0, e1) * 1e3 / 100, 2)
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
              "decode_us_per_step_across_g_boundaries": boundary,
              "decode_plain_us_per_step_at_those_lengths": boundary_plain}
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
        wsb = torch.empty(max(16, jl.decode_batch_workspace_bytes(lens, Hq, Hkv)), dtype=torch.uint8, device=dev)

        def step():
            jl.decode_batch(qb, kb_, vb, lens, row0=row0, w0=dcfg.w0, w_pretrained=dcfg.w_pretrained,
                            rope_base=dcfg.rope_base, out=ob, lse=lb, workspace=wsb)

        for _ in range(4):
            step()
        torch.cuda.synchronize()
        n = 50
        ev.record(e0, stream)
        for _ in range(n):
            step()
        ev.record(e1, stream)
        us = ev.elapsed_ms(e0, e1) * 1e3 / n
        torch.cuda.synchronize()
        kvb = 2 * sum(lens) * Hkv * d * 2
        log(f"[bench] batched decode of {len(lens)} sequences: {us:.1f} us per step ({kvb / us / 1e3:.0f} GB/s)")
        return {"lens": lens, "us_per_step": round(us, 2), "kv_bytes": kvb,
                "GB/s": round(kvb / (us * 1e-6) / 1e9, 1), "frac_hbm": round(kvb / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}

    dj_obj, ov_obj = (None, None) if args.headline_only else run_extras()
    db_obj = None if args.headline_only else run_decode_batch()

    tflops = F3 / (call_ms * 1e-3) / 1e12
    pass2_tflops = Fc / (pass2_ms * 1e-3) / 1e12
    dec_gbs = kv_bytes / (dec_us * 1e-6) / 1e9
    log(f"[bench] prefill call {call_ms:.2f} ms -> {tflops:.1f} TFLOP/s (F_3pass); attention kernels "
        f"{attn_ms:.2f} ms; pass 2 {pass2_ms:.2f} ms -> {pass2_tflops:.1f} TFLOP/s; decode {dec_us:.1f} "
        f"us/step ({dec_gbs:.0f} GB/s)")

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
        "roofline": {"bound": "mfma", "achieved": round(pass2_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(pass2_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": read_traffic(PASS2_TRAFFIC),
                     "kernel": "prefill_pp_kernel<0> + prefill_pass_kernel<0, true> (pass 2: remote "
                               "q/k, full causal; the second kernel takes the first 128 rows)",
                     "flops_per_launch": Fc, "ms_per_launch": round(pass2_ms, 3)},
        "prefill": {"call_ms": round(call_ms, 3), "attention_ms": round(attn_ms, 3),
                    "pass2_ms": round(pass2_ms, 3), "tflops_3pass": round(tflops, 2),
                    "tflops_causal_basis": round(Fc / (call_ms * 1e-3) / 1e12, 2),
                    "flops_3pass": F3, "flops_causal": Fc},
        "decode": {"us_per_step": round(dec_us, 2), "us_in_step": round(dec_in_step_us, 2),
                   "kv_bytes": kv_bytes, "GB/s": round(dec_gbs, 1),
                   "roofline": {"bound": "hbm", "achieved": round(dec_gbs, 1), "peak": PEAK_HBM_GBS,
                                "unit": "GB/s", "frac": round(dec_gbs / PEAK_HBM_GBS, 4),
                                "traffic": read_traffic(DECODE_TRAFFIC),
                                "kernel": "decode_split_kernel + decode_reduce_kernel (one step, timed "
                                          "over back-to-back steps)", "us_per_launch": round(dec_us, 2)},
                   "step_frac_hbm": round(dec_gbs / PEAK_HBM_GBS, 4)},
        "disjoint_merge": dj_obj,
        "overhead": ov_obj,
        "decode_batch": db_obj,
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
