"""Ragged multi-sequence decode (one call, B sequences with their own L, G,
query and cache rows) against the fp64 oracle's single-sequence decode of
every sequence, and against the library's own single-sequence decode.  Every
sequence follows the technical summary, Methodology item 2 on its own: its
cache holds base keys at their absolute positions and its correction
rotation depends on its own length."""

import sys

import numpy as np
import pytest

import oracle
import workloads as W
from jl_testutil import BF16_LSE_RTOL, BF16_O_ATOL, gpu_or_skip, lse_rel_err, max_abs

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _check_against_oracle(q, kc, vc, row0, lens, o, lse, seqs, w0, wpt, base, q_to_kv=None):
    worst_o = worst_l = 0.0
    for b in seqs:
        L, r = lens[b], row0[b]
        oo, ll = oracle.decode(q[b].double().numpy(), kc[r:r + L].double().numpy(), vc[r:r + L].double().numpy(),
                               L, w0=w0, w_pretrained=wpt, rope_base=base, q_to_kv=q_to_kv)
        e_o, e_l = max_abs(o[b], oo), lse_rel_err(lse[b], ll)
        _say(f"[decode-batch] seq {b} L={L} G={oracle.group_size(L, wpt)}: max|do|={e_o:.3e} lse rel={e_l:.3e}")
        worst_o, worst_l = max(worst_o, e_o), max(worst_l, e_l)
    assert worst_o <= BF16_O_ATOL
    assert worst_l <= BF16_LSE_RTOL


def test_ragged_batch_matches_oracle():
    """Qwen3-8B heads; lengths on both sides of the G boundary at 32768, one
    empty sequence (its outputs stay untouched), spare rows between the
    sequences' cache ranges."""
    jl, torch = gpu_or_skip()
    lens = [1, 63, 65, 4097, 0, 32768, 32769, 20000]
    Hq, Hkv, w0, wpt, base = 32, 8, 4096, 32768, 1e6
    q, kc, vc, row0 = W.make_decode_batch_inputs(Hq, Hkv, 128, lens, seed=41, gap=37)
    _say(f"[decode-batch] lens={lens} rows={kc.shape[0]}")
    qd, kd, vd = q.cuda(), kc.cuda(), vc.cuda()
    k_before, v_before = kd.clone(), vd.clone()
    o = torch.full_like(qd, 7.0)
    lse = torch.full((len(lens), Hq), 7.0, device="cuda")
    jl.decode_batch(qd, kd, vd, lens, row0=row0, w0=w0, w_pretrained=wpt, rope_base=base, out=o, lse=lse)
    torch.cuda.synchronize()
    # the caches are never written: every bit is unchanged
    assert torch.equal(kd.view(torch.int16), k_before.view(torch.int16))
    assert torch.equal(vd.view(torch.int16), v_before.view(torch.int16))
    og, lg = o.float().cpu().numpy(), lse.cpu().numpy()
    assert np.all(og[4] == 7.0) and np.all(lg[4] == 7.0)                    # L = 0: not written
    _check_against_oracle(q, kc, vc, row0, lens, og, lg, [b for b in range(len(lens)) if lens[b]], w0, wpt, base)


def test_small_heads_shared_rows_and_head_map():
    """8 q / 2 kv heads with an explicit head map, G from 1 to 4, and two
    sequences that read the same cache rows (the first a prefix of the
    second)."""
    jl, torch = gpu_or_skip()
    lens = [3, 300, 1000, 129, 500, 700]
    Hq, Hkv, w0, wpt, base = 8, 2, 100, 256, 1e4
    kvmap = [1, 0, 1, 0, 0, 1, 1, 0]
    q, kc, vc, row0 = W.make_decode_batch_inputs(Hq, Hkv, 128, lens, seed=43, gap=5)
    row0[5] = row0[4]                       # sequence 5 extends sequence 4's rows
    kc, vc = kc[:row0[4] + 700 + 5], vc[:row0[4] + 700 + 5]
    o, lse = jl.decode_batch(q.cuda(), kc.cuda(), vc.cuda(), lens, row0=row0, w0=w0, w_pretrained=wpt,
                             rope_base=base, q_to_kv=kvmap)
    torch.cuda.synchronize()
    _check_against_oracle(q, kc, vc, row0, lens, o.float().cpu().numpy(), lse.cpu().numpy(), range(len(lens)),
                          w0, wpt, base, q_to_kv=kvmap)


@pytest.mark.parametrize("Hq,Hkv", [(8, 8), (16, 2), (3, 3)])
def test_batch_group_sizes(Hq, Hkv):
    """1, 8 and 1 (with three kv heads: a wave without a kv head) q heads per
    kv head; ragged lengths with G from 1 to 5."""
    jl, torch = gpu_or_skip()
    lens = [700, 1, 2049, 333, 1500]
    w0, wpt, base = 128, 400, 1e4
    q, kc, vc, row0 = W.make_decode_batch_inputs(Hq, Hkv, 128, lens, seed=Hq * 10 + Hkv, gap=3)
    o, lse = jl.decode_batch(q.cuda(), kc.cuda(), vc.cuda(), lens, row0=row0, w0=w0, w_pretrained=wpt,
                             rope_base=base)
    torch.cuda.synchronize()
    _check_against_oracle(q, kc, vc, row0, lens, o.float().cpu().numpy(), lse.cpu().numpy(), range(len(lens)),
                          w0, wpt, base)


def test_one_sequence_is_the_single_call():
    """A batch of one runs the same plan as jl_bifocal_decode: same bits."""
    jl, torch = gpu_or_skip()
    cfg = W.decode_8b(65537)
    q, kc, vc = W.make_decode_inputs(cfg)
    qd, kd, vd = q.cuda(), kc.cuda(), vc.cuda()
    kw = dict(w0=cfg.w0, w_pretrained=cfg.w_pretrained, rope_base=cfg.rope_base)
    o1, l1 = jl.decode(qd, kd, vd, cfg.L, **kw)
    ob, lb = jl.decode_batch(qd[None], kd, vd, [cfg.L], **kw)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), ob[0].view(torch.int16))
    assert torch.equal(l1, lb[0])


def test_varlen_8_sequences_8k_to_128k():
    """Eight sequences with the Qwen3-4B varlen lengths (8K .. 128K, seeded),
    32 q / 8 kv heads: every sequence against the library's single-sequence
    decode, the shortest and the longest against the oracle."""
    jl, torch = gpu_or_skip()
    lens = list(W.varlen_4b(4096).seqlens)
    Hq, Hkv, w0, wpt, base = 32, 8, 4096, 32768, 1e6
    q, kc, vc, row0 = W.make_decode_batch_inputs(Hq, Hkv, 128, lens, seed=47, device="cuda")
    _say(f"[decode-batch] lens={lens} rows={kc.shape[0]}")
    kw = dict(w0=w0, w_pretrained=wpt, rope_base=base)
    o, lse = jl.decode_batch(q, kc, vc, lens, row0=row0, **kw)
    torch.cuda.synchronize()
    worst_o = worst_l = 0.0
    for b, L in enumerate(lens):
        r = row0[b]
        os_, ls_ = jl.decode(q[b], kc[r:r + L], vc[r:r + L], L, **kw)
        torch.cuda.synchronize()
        worst_o = max(worst_o, (o[b].float() - os_.float()).abs().max().item())
        worst_l = max(worst_l, lse_rel_err(lse[b].cpu().numpy(), ls_.cpu().numpy()))
    _say(f"[decode-batch] vs single-sequence calls: max|do|={worst_o:.3e} lse rel={worst_l:.3e}")
    assert worst_o <= BF16_O_ATOL and worst_l <= BF16_LSE_RTOL
    check = [lens.index(min(lens)), lens.index(max(lens))]
    qc, og, lg = q.cpu(), o.float().cpu().numpy(), lse.cpu().numpy()
    for b in check:
        r, L = row0[b], lens[b]
        oo, ll = oracle.decode(qc[b].double().numpy(), kc[r:r + L].cpu().double().numpy(),
                               vc[r:r + L].cpu().double().numpy(), L, **kw)
        e_o, e_l = max_abs(og[b], oo), lse_rel_err(lg[b], ll)
        _say(f"[decode-batch] seq {b} L={L}: max|do|={e_o:.3e} lse rel={e_l:.3e}")
        assert e_o <= BF16_O_ATOL and e_l <= BF16_LSE_RTOL


def test_batch_repeated_calls_are_bitwise_identical():
    jl, torch = gpu_or_skip()
    lens = list(W.varlen_4b(4096).seqlens)[:4]
    q, kc, vc, row0 = W.make_decode_batch_inputs(32, 8, 128, lens, seed=53, device="cuda")
    kw = dict(row0=row0, w0=4096, w_pretrained=32768, rope_base=1e6)
    o0, l0 = jl.decode_batch(q, kc, vc, lens, **kw)
    for _ in range(3):
        o, l = jl.decode_batch(q, kc, vc, lens, **kw)
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), o0.view(torch.int16))
        assert torch.equal(l, l0)


def test_batch_max_sequences():
    """JL_MAX_SEQS (64) sequences of seeded lengths 0 .. 3000 in one call."""
    jl, torch = gpu_or_skip()
    g = torch.Generator("cpu").manual_seed(73)
    lens = [int(x) for x in torch.randint(0, 3001, (64,), generator=g)]
    lens[3] = 0
    lens[4] = 1
    Hq, Hkv, w0, wpt, base = 8, 2, 200, 700, 1e4
    q, kc, vc, row0 = W.make_decode_batch_inputs(Hq, Hkv, 128, lens, seed=74, gap=1)
    o = torch.zeros((64, Hq, 128), dtype=torch.bfloat16, device="cuda")
    o, lse = jl.decode_batch(q.cuda(), kc.cuda(), vc.cuda(), lens, row0=row0, w0=w0, w_pretrained=wpt,
                             rope_base=base, out=o)
    torch.cuda.synchronize()
    _check_against_oracle(q, kc, vc, row0, lens, o.float().cpu().numpy(), lse.cpu().numpy(),
                          [b for b in range(64) if lens[b]], w0, wpt, base)


def test_batch_decode_on_the_packed_prefill_cache():
    """Packed varlen prefill that writes its keys' cache, then one batched
    decode step per sequence straight on that packed cache (row0 =
    cu_seqlens): each sequence's step at L = its length must equal the last
    row of its prefill, against the fp64 oracle (bf16 bars) and against the
    library's prefill row (twice the bars: both within the bar of the
    oracle)."""
    jl, torch = gpu_or_skip()
    Hq, Hkv, d, w0, wpt, base = 8, 2, 128, 96, 300, 1e6
    lens = [250, 700, 1200, 301]                       # G = 1, 3, 4, 2
    cu = [0]
    for n in lens:
        cu.append(cu[-1] + n)
    T = cu[-1]
    g = torch.Generator("cpu").manual_seed(29)
    q = torch.randn((T, Hq, d), generator=g).bfloat16()
    k = torch.randn((T, Hkv, d), generator=g).bfloat16()
    v = torch.randn((T, Hkv, d), generator=g).bfloat16()
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    kc = torch.empty((T, Hkv, d), dtype=torch.bfloat16, device="cuda")
    o_p, lse_p = jl.prefill(qd, kd, vd, w0=w0, w_pretrained=wpt, rope_base=base, cu_seqlens=cu, k_cache_out=kc)
    # the newest query of each sequence, base-rotated at its position L_b - 1
    qlast = torch.stack([jl.rope_rows(qd[cu[b + 1] - 1:cu[b + 1]], lens[b] - 1, rope_base=base)[0]
                         for b in range(len(lens))])
    o_d, lse_d = jl.decode_batch(qlast, kc, vd, lens, row0=cu[:-1], w0=w0, w_pretrained=wpt, rope_base=base)
    torch.cuda.synchronize()
    for b, n in enumerate(lens):
        s0, s1 = cu[b], cu[b + 1]
        oo, ll = oracle.prefill(q[s0:s1].double().numpy(), k[s0:s1].double().numpy(), v[s0:s1].double().numpy(),
                                w0=w0, w_pretrained=wpt, rope_base=base, rows=[n - 1])
        od, ld = o_d[b].float().cpu().numpy(), lse_d[b].cpu().numpy()
        e_o, e_l = max_abs(od, oo[0]), lse_rel_err(ld, ll[:, 0])
        _say(f"[prefill->batch] seq {b} L={n} G={jl.group_size(n, wpt)}: vs oracle max|do|={e_o:.3e} "
             f"lse rel={e_l:.3e}")
        assert e_o <= BF16_O_ATOL and e_l <= BF16_LSE_RTOL
        assert max_abs(od, o_p[s1 - 1].float().cpu().numpy()) <= 2 * BF16_O_ATOL
        assert lse_rel_err(ld, lse_p[:, s1 - 1].cpu().numpy()) <= 2 * BF16_LSE_RTOL


def test_decode_past_one_round_of_partials():
    """A sequence longer than 256 workgroups of the largest sub-chunk count
    (256 x 65536 keys) leaves the merge more partials per head than it takes
    in one round (256).  With w0 >= L every key takes the base path and no
    position enters a score, so softmax attention over all keys must equal
    the LSE merge of one batched call over two halves of the keys, whose
    merges take one round each.  Planted keys (one per 65536-key workgroup,
    scores about 9 to 12 above the others' unit spread) carry most of the
    softmax mass, so the output depends on the weight of every partial."""
    jl, torch = gpu_or_skip()
    Hq, Hkv, d, base, wpt = 4, 1, 128, 1e6, 32768
    L = 259 * 65536 - 5
    L1 = 130 * 65536 + 12345                            # inside a workgroup's range
    _say(f"[decode-long] L={L} halves {L1} + {L - L1}")
    g = torch.Generator(device="cuda").manual_seed(61)
    q = torch.randn((Hq, d), generator=g, device="cuda")
    kc = torch.randn((L, Hkv, d), generator=g, device="cuda").bfloat16()
    vc = torch.randn((L, Hkv, d), generator=g, device="cuda").bfloat16()
    qn = (q / q.norm(dim=1, keepdim=True)).sum(0)       # scores about c for every head
    for w in range(259):
        j = 65536 * w + (1000 + 37 * w) % 60000
        c = 9.0 + 0.75 * ((7 * w) % 5)
        kc[j, 0] = (c * qn).bfloat16()
        vc[j, 0] = torch.randn((d,), generator=g, device="cuda").bfloat16()
    qb = q.bfloat16()
    kw = dict(w0=L, w_pretrained=wpt, rope_base=base)
    o, lse = jl.decode(qb, kc, vc, L, **kw)
    oh, lh = jl.decode_batch(torch.stack([qb, qb]), kc, vc, [L1, L - L1], row0=[0, L1], **kw)
    torch.cuda.synchronize()
    oh, lh = oh.double().cpu(), lh.double().cpu()
    M = lh.max(dim=0).values
    z = torch.exp(lh - M)                               # [2, Hq]
    o_ref = (z[:, :, None] * oh).sum(0) / z.sum(0)[:, None]
    lse_ref = M + torch.log(z.sum(0))
    og, lg = o.double().cpu(), lse.double().cpu()
    e_o = (og - o_ref).abs().max().item()
    e_l = (lg - lse_ref).abs().max().item()
    scale_o = o_ref.abs().max().item()
    _say(f"[decode-long] max|O| {scale_o:.3f}, max|dO| {e_o:.2e}, max|dlse| {e_l:.2e}, "
         f"half masses {z[0].mean().item():.3f} / {z[1].mean().item():.3f}")
    assert 0.1 < scale_o < 10.0                         # the planted keys dominate the output (0.265 seen)
    assert e_o <= 1e-2 * scale_o                        # two bf16 roundings of the halves, one of the whole
    assert e_l <= 1e-4                                  # fp32 sums over 17M keys, natural-log units
