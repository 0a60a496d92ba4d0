// jl_api.hip - the C ABI of libjetlong.so: argument validation, workspace
// protocol and dispatch onto the caller's HIP stream.  See include/jetlong.h.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "../../include/jetlong_testing.h"
#include "jl_internal.h"

#define JL_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

thread_local char g_err[256] = "";
thread_local hipEvent_t g_ev_before = nullptr, g_ev_mid = nullptr, g_ev_after = nullptr;

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(JL_EHIP, "%s: %s", what, hipGetErrorString(e));
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// theta_m / (2 pi) modulo 1 in unsigned 0.64 fixed point, from long double.
// Only the fractional part matters: p * (n + f) = p * f modulo a whole turn.
void build_freqs(JlFreqs* fr, int d, double base) {
  const long double two_pi = 6.283185307179586476925286766559005768L;
  for (int m = 0; m < d / 2; ++m) {
    const long double theta = powl((long double)base, -(long double)(2 * m) / (long double)d);
    long double f = fmodl(theta / two_pi, 1.0L);
    if (f < 0) f += 1.0L;
    fr->turn_frac[m] = (uint64_t)ldexpl(f, 64) ;
  }
  for (int m = d / 2; m < JL_MAX_HALF; ++m) fr->turn_frac[m] = 0;
}

// The table for (d, base), built once per thread: 64 long double
// pow/fmod/ldexp evaluations cost more host time than a short decode step
// takes on the GPU, and a generation loop asks for the same table every step.
const JlFreqs& freqs_for(int d, double base) {
  thread_local int c_d = -1;
  thread_local double c_base = 0.0;
  thread_local JlFreqs c_fr;
  if (c_d != d || c_base != base) {
    build_freqs(&c_fr, d, base);
    c_d = d;
    c_base = base;
  }
  return c_fr;
}

int build_head_map(JlHeadMap* hm, int Hq, int Hkv, const int32_t* q_to_kv) {
  if (Hq < 1 || Hkv < 1) return fail(JL_EINVAL, "num_q_heads and num_kv_heads must be >= 1");
  if (Hq > JL_MAX_HEADS) return fail(JL_EUNSUPPORTED, "num_q_heads > %d", JL_MAX_HEADS);
  if (Hkv > Hq) return fail(JL_EINVAL, "num_kv_heads > num_q_heads");
  if (q_to_kv == nullptr) {
    if (Hq % Hkv) return fail(JL_EINVAL, "num_q_heads %% num_kv_heads != 0 and no q_to_kv map", 0);
    for (int h = 0; h < Hq; ++h) hm->kv_of[h] = (uint8_t)(h / (Hq / Hkv));
  } else {
    for (int h = 0; h < Hq; ++h) {
      if (q_to_kv[h] < 0 || q_to_kv[h] >= Hkv) return fail(JL_EINVAL, "q_to_kv[%d] out of range", h);
      hm->kv_of[h] = (uint8_t)q_to_kv[h];
    }
  }
  for (int h = Hq; h < JL_MAX_HEADS; ++h) hm->kv_of[h] = 0;
  for (int h = 0; h < JL_MAX_HEADS; ++h) hm->head_of_slot[h] = 0;
  if (Hq % Hkv == 0) {
    const int NG = Hq / Hkv;
    int cnt[JL_MAX_HEADS] = {0};
    for (int h = 0; h < Hq; ++h) {
      const int kv = hm->kv_of[h];
      if (cnt[kv] < NG) hm->head_of_slot[kv * NG + cnt[kv]] = (uint8_t)h;
      ++cnt[kv];
    }
  }
  return JL_OK;
}

int check_common(int64_t w0, int64_t w_pretrained, double rope_base) {
  if (w0 < 0) return fail(JL_EINVAL, "w0 must be >= 0");
  if (w_pretrained < 1) return fail(JL_EINVAL, "w_pretrained must be >= 1");
  if (!(rope_base > 0.0) || !isfinite(rope_base)) return fail(JL_EINVAL, "rope_base must be finite and > 0");
  return JL_OK;
}

// The device-shape cache: one entry per device, filled once under its flag.
constexpr int JL_MAX_DEVICES = 64;
std::once_flag g_shape_once[JL_MAX_DEVICES];
JlDevShape g_shape[JL_MAX_DEVICES];
const JlDevShape kDefaultShape{256, 8};   // a full MI355X: 256 CUs in 8 XCDs of 32

JlDevShape read_device_shape(int dev) {
  JlDevShape s = kDefaultShape;
  int cus = 0, xccs = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    return s;
  s.cus = cus;
  // XCD count as the runtime reports it; gfx950 has 32 CUs per XCD in every
  // partition mode, which serves when the attribute is missing
  if (hipDeviceGetAttribute(&xccs, hipDeviceAttributeNumberOfXccs, dev) == hipSuccess && xccs >= 1)
    s.xcds = xccs;
  else
    s.xcds = cus >= 32 ? cus / 32 : 1;
  return s;
}

struct PrefillPlan {
  JlSeqs seqs;
  int32_t max_len;
  int64_t t_pad;
  size_t off_qb, off_qr, off_kb, off_kr, off_vt, off_lo, off_o, off_lse, total;
};

}  // namespace

JlDevShape jl_device_shape() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= JL_MAX_DEVICES) {
    (void)hipGetLastError();   // no device on this host: clear the sticky error
    return kDefaultShape;
  }
  std::call_once(g_shape_once[dev], [dev] { g_shape[dev] = read_device_shape(dev); });
  return g_shape[dev];
}

JL_EXPORT int64_t jl_group_size(int64_t L, int64_t w_pretrained) {
  if (L < 0 || w_pretrained < 1) return fail(JL_EINVAL, "jl_group_size needs L >= 0 and w_pretrained >= 1");
  return jl_group_size_i64(L, w_pretrained);
}

JL_EXPORT const char* jl_last_error(void) { return g_err; }

static int prefill_impl(const void* q, const void* k, const void* v, void* o, float* lse,
                        const int64_t* cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                        int32_t num_q_heads, int32_t num_kv_heads, const int32_t* q_to_kv,
                        int32_t head_dim, jl_dtype dtype, int64_t w0, int64_t w_pretrained,
                        double rope_base, float softmax_scale, void* workspace,
                        size_t* workspace_bytes, void* hip_stream, bool disjoint, void* k_cache) {
  if (workspace_bytes == nullptr) return fail(JL_EINVAL, "workspace_bytes is NULL");
  if (total_tokens < 0) return fail(JL_EINVAL, "total_tokens < 0");
  if (dtype != JL_BF16 && dtype != JL_FP32) return fail(JL_EINVAL, "unknown dtype %d", (int)dtype);
  int rc = check_common(w0, w_pretrained, rope_base);
  if (rc) return rc;
  JlHeadMap hm;
  rc = build_head_map(&hm, num_q_heads, num_kv_heads, q_to_kv);
  if (rc) return rc;
  if (disjoint && dtype != JL_BF16) return fail(JL_EUNSUPPORTED, "the disjoint merge is built for bf16 only");
  if (dtype == JL_BF16 && head_dim != 128) return fail(JL_EUNSUPPORTED, "bf16 prefill needs head_dim 128");
  if (dtype == JL_FP32 && head_dim != 64 && head_dim != 128)
    return fail(JL_EUNSUPPORTED, "fp32 prefill needs head_dim 64 or 128");
  if (num_seqs < 1) return fail(JL_EINVAL, "num_seqs must be >= 1");
  if (num_seqs > JL_MAX_SEQS) return fail(JL_EUNSUPPORTED, "num_seqs > %d", JL_MAX_SEQS);
  if (cu_seqlens == nullptr && num_seqs != 1) return fail(JL_EINVAL, "cu_seqlens is NULL with num_seqs > 1");
  if (total_tokens > (int64_t)INT32_MAX - 512) return fail(JL_EUNSUPPORTED, "total_tokens too large");

  PrefillPlan pl;
  memset(&pl, 0, sizeof(pl));
  pl.seqs.nseq = num_seqs;
  for (int b = 0; b < num_seqs; ++b) {
    int64_t s0 = cu_seqlens ? cu_seqlens[b] : 0;
    int64_t s1 = cu_seqlens ? cu_seqlens[b + 1] : total_tokens;
    if (b == 0 && s0 != 0) return fail(JL_EINVAL, "cu_seqlens[0] != 0");
    if (s1 < s0) return fail(JL_EINVAL, "cu_seqlens decreases at %d", b);
    // the bf16 pass kernels copy a sequence's K and V tiles through buffer
    // resources with 31-bit byte offsets: 256 bytes per key, tiles of 64 keys
    if (dtype == JL_BF16 && s1 - s0 > JL_BF16_MAX_SEQ_LEN)
      return fail(JL_EUNSUPPORTED, "bf16 prefill supports sequences of up to %lld tokens (sequence %d has %lld)",
                  (long long)JL_BF16_MAX_SEQ_LEN, b, (long long)(s1 - s0));
    // the fp32 kernel runs one 64-lane workgroup per row of a sequence
    if (dtype == JL_FP32 && s1 - s0 > JL_FP32_MAX_SEQ_LEN)
      return fail(JL_EUNSUPPORTED, "fp32 prefill supports sequences of up to %lld tokens (sequence %d has %lld)",
                  (long long)JL_FP32_MAX_SEQ_LEN, b, (long long)(s1 - s0));
    pl.seqs.start[b] = (int32_t)s0;
    pl.seqs.len[b] = (int32_t)(s1 - s0);
    pl.seqs.G[b] = (int32_t)jl_group_size_i64(s1 - s0, w_pretrained);
    if (pl.seqs.G[b] > 1) pl.seqs.any_remote = 1;
    if (pl.seqs.len[b] > pl.max_len) pl.max_len = pl.seqs.len[b];
    pl.seqs.vstart[b] = pl.seqs.vt_cols;
    pl.seqs.vt_cols += (pl.seqs.len[b] + 63) / 64 * 64;
  }
  if (cu_seqlens && cu_seqlens[num_seqs] != total_tokens)
    return fail(JL_EINVAL, "cu_seqlens[num_seqs] != total_tokens");

  const size_t el = dtype == JL_BF16 ? 2 : 4;
  pl.t_pad = jl_prefill_t_pad(total_tokens);
  const size_t nq = (size_t)num_q_heads * pl.t_pad * head_dim * el;
  const size_t nk = (size_t)num_kv_heads * pl.t_pad * head_dim * el;
  size_t off = 0;
  // the bf16 kernels rotate q themselves: only the fp32 path keeps rotated q
  const bool q_in_ws = dtype != JL_BF16;
  pl.off_qb = off; if (q_in_ws) off += align256(nq);
  pl.off_qr = off; if (q_in_ws && pl.seqs.any_remote) off += align256(nq);
  pl.off_kb = off; off += align256(nk);
  pl.off_kr = off; if (pl.seqs.any_remote) off += align256(nk);
  pl.off_vt = off;
  if (dtype == JL_BF16) off += align256((size_t)num_kv_heads * head_dim * pl.seqs.vt_cols * el);
  // split-operand residuals of k's first JL_LO_ROWS positions (bf16 path; the
  // kernels form q's residuals from q)
  const size_t lrows = (size_t)num_seqs * JL_LO_ROWS;
  const size_t nklo = (size_t)num_kv_heads * lrows * head_dim * el;
  pl.off_lo = off; if (dtype == JL_BF16) off += 2 * align256(nklo);
  // rows >= JL_LO_ROWS: the three-pass kernel keeps pass 3's state
  // (accumulator, stabiliser and sum) until it has formed the far part; the
  // accumulator takes those rows of the o2 array, which only the disjoint
  // variant's far pass uses otherwise (one or the other per call), and a
  // sequence's first JL_LO_ROWS rows of o2 hold pass 2's output for the
  // launch that runs pass 3 and merges them
  const bool merge = dtype == JL_BF16 && pl.seqs.any_remote;
  const size_t no = align256((size_t)num_q_heads * total_tokens * head_dim * 4);
  const size_t nl = align256((size_t)num_q_heads * total_tokens * 4);
  const size_t no1 = align256((size_t)num_q_heads * lrows * head_dim * 4);
  const size_t nl1 = align256((size_t)num_q_heads * lrows * 4);
  pl.off_o = off; if (merge) off += no1 + no;
  pl.off_lse = off; if (merge) off += nl1 + 3 * nl;
  pl.total = total_tokens == 0 ? 0 : off;

  if (workspace == nullptr) {
    *workspace_bytes = pl.total;
    return JL_OK;
  }
  if (*workspace_bytes < pl.total)
    return fail(JL_ENOSPC, "workspace has %zu bytes, %zu needed", *workspace_bytes, pl.total);
  if (total_tokens == 0) return JL_OK;
  if (!q || !k || !v || !o) return fail(JL_EINVAL, "q, k, v and o must be device pointers");
  if (((uintptr_t)workspace & 255) != 0) return fail(JL_EINVAL, "workspace must be 256-byte aligned");
  if (dtype == JL_BF16 && (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15))
    return fail(JL_EINVAL, "bf16 tensors must be 16-byte aligned");
  if (k_cache != nullptr && ((uintptr_t)k_cache & 15)) return fail(JL_EINVAL, "k_cache must be 16-byte aligned");

  const JlFreqs& fr = freqs_for(head_dim, rope_base);
  const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf((float)head_dim);
  hipStream_t st = (hipStream_t)hip_stream;
  char* wsb = (char*)workspace;
  JlPrefillWs ws;
  ws.qb = q_in_ws ? (void*)(wsb + pl.off_qb) : nullptr;
  ws.qr = q_in_ws && pl.seqs.any_remote ? (void*)(wsb + pl.off_qr) : ws.qb;
  ws.kb = wsb + pl.off_kb;
  ws.kr = pl.seqs.any_remote ? (void*)(wsb + pl.off_kr) : ws.kb;
  ws.vt = dtype == JL_BF16 ? (void*)(wsb + pl.off_vt) : nullptr;
  ws.kb_lo = ws.kr_lo = nullptr;
  ws.kc = k_cache;
  {
    const size_t lrows = (size_t)num_seqs * JL_LO_ROWS;
    const size_t no1 = align256((size_t)num_q_heads * lrows * head_dim * 4);
    const size_t nl1 = align256((size_t)num_q_heads * lrows * 4);
    const size_t nl = align256((size_t)num_q_heads * total_tokens * 4);
    ws.o1 = wsb + pl.off_o;
    ws.o2 = wsb + pl.off_o + no1;
    ws.o3 = ws.o2;   // rows >= JL_LO_ROWS only (see the layout above)
    ws.lse1 = wsb + pl.off_lse;
    ws.lse2 = wsb + pl.off_lse + nl1;
    ws.ml3 = wsb + pl.off_lse + nl1 + nl;
  }
  if (dtype == JL_BF16) {
    const size_t lrows = (size_t)num_seqs * JL_LO_ROWS;
    const size_t nklo = align256((size_t)num_kv_heads * lrows * head_dim * el);
    ws.kb_lo = wsb + pl.off_lo;
    ws.kr_lo = pl.seqs.any_remote ? (void*)(wsb + pl.off_lo + nklo) : ws.kb_lo;   // one grid: shared
  }
  ws.t_pad = pl.t_pad;

  // the bf16 kernels take q pre-multiplied by scale * log2(e)
  const float qscale = dtype == JL_BF16 ? scale * 1.4426950408889634f : 1.f;
  hipError_t e = jl_launch_rope_prepass(q, k, ws, (int)el, total_tokens, q_in_ws ? num_q_heads : 0,
                                        num_kv_heads, head_dim, pl.seqs, fr, qscale, st);
  if (e != hipSuccess) return hip_fail(e, "rope pre-pass launch");
  if (dtype == JL_BF16) {
    e = jl_launch_transpose_v(v, ws, pl.seqs, num_kv_heads, st);
    if (e != hipSuccess) return hip_fail(e, "v transpose launch");
    if (g_ev_before) (void)hipEventRecord(g_ev_before, st);
    e = jl_launch_prefill_bf16(ws, q, fr, qscale, o, lse, total_tokens, num_q_heads, num_kv_heads, hm,
                               pl.seqs, w0, scale, pl.max_len, disjoint, st);
    if (e != hipSuccess) return hip_fail(e, "bf16 prefill launch");
    if (g_ev_after) (void)hipEventRecord(g_ev_after, st);
  } else {
    if (g_ev_before) (void)hipEventRecord(g_ev_before, st);
    e = jl_launch_prefill_fp32(ws, (const float*)v, (float*)o, lse, total_tokens, num_q_heads,
                               num_kv_heads, head_dim, hm, pl.seqs, w0, scale, pl.max_len, st);
    if (e != hipSuccess) return hip_fail(e, "fp32 prefill launch");
    if (g_ev_after) (void)hipEventRecord(g_ev_after, st);
  }
  return JL_OK;
}

JL_EXPORT int jl_bifocal_prefill(const void* q, const void* k, const void* v, void* o, float* lse,
                                 const int64_t* cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                                 int32_t num_q_heads, int32_t num_kv_heads, const int32_t* q_to_kv,
                                 int32_t head_dim, jl_dtype dtype, int64_t w0, int64_t w_pretrained,
                                 double rope_base, float softmax_scale, void* workspace,
                                 size_t* workspace_bytes, void* hip_stream) {
  return prefill_impl(q, k, v, o, lse, cu_seqlens, num_seqs, total_tokens, num_q_heads, num_kv_heads, q_to_kv,
                      head_dim, dtype, w0, w_pretrained, rope_base, softmax_scale, workspace, workspace_bytes,
                      hip_stream, false, nullptr);
}

JL_EXPORT int jl_bifocal_prefill_kcache(const void* q, const void* k, const void* v, void* o, float* lse,
                                        void* k_cache, const int64_t* cu_seqlens, int32_t num_seqs,
                                        int64_t total_tokens, int32_t num_q_heads, int32_t num_kv_heads,
                                        const int32_t* q_to_kv, int32_t head_dim, jl_dtype dtype, int64_t w0,
                                        int64_t w_pretrained, double rope_base, float softmax_scale,
                                        void* workspace, size_t* workspace_bytes, void* hip_stream) {
  if (k_cache == nullptr && workspace != nullptr && total_tokens > 0)
    return fail(JL_EINVAL, "k_cache must be a device pointer");
  return prefill_impl(q, k, v, o, lse, cu_seqlens, num_seqs, total_tokens, num_q_heads, num_kv_heads, q_to_kv,
                      head_dim, dtype, w0, w_pretrained, rope_base, softmax_scale, workspace, workspace_bytes,
                      hip_stream, false, k_cache);
}

JL_EXPORT int jl_bifocal_prefill_disjoint(const void* q, const void* k, const void* v, void* o, float* lse,
                                          const int64_t* cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                                          int32_t num_q_heads, int32_t num_kv_heads, const int32_t* q_to_kv,
                                          int32_t head_dim, jl_dtype dtype, int64_t w0, int64_t w_pretrained,
                                          double rope_base, float softmax_scale, void* workspace,
                                          size_t* workspace_bytes, void* hip_stream) {
  return prefill_impl(q, k, v, o, lse, cu_seqlens, num_seqs, total_tokens, num_q_heads, num_kv_heads, q_to_kv,
                      head_dim, dtype, w0, w_pretrained, rope_base, softmax_scale, workspace, workspace_bytes,
                      hip_stream, true, nullptr);
}

// One or more sequences: lens[b] keys at cache rows row0[b] .. row0[b] + lens[b] - 1.
// cache_rows < 0: the caller gave no cache size (single-sequence call).
static int decode_impl(const void* q, const void* k_cache, const void* v_cache, int64_t cache_rows,
                       const int64_t* row0, const int64_t* lens, int32_t num_seqs, void* o, float* lse,
                       int32_t num_q_heads, int32_t num_kv_heads, const int32_t* q_to_kv, int32_t head_dim,
                       jl_dtype dtype, int64_t w0, int64_t w_pretrained, double rope_base, float softmax_scale,
                       void* workspace, size_t* workspace_bytes, void* hip_stream) {
  if (workspace_bytes == nullptr) return fail(JL_EINVAL, "workspace_bytes is NULL");
  if (num_seqs < 1) return fail(JL_EINVAL, "num_seqs must be >= 1");
  if (num_seqs > JL_MAX_SEQS) return fail(JL_EUNSUPPORTED, "num_seqs > %d", JL_MAX_SEQS);
  if (lens == nullptr || row0 == nullptr) return fail(JL_EINVAL, "lens and row0 must be host arrays");
  int64_t total = 0;
  for (int b = 0; b < num_seqs; ++b) {
    if (lens[b] < 0) return fail(JL_EINVAL, "L < 0 (sequence %d)", b);
    if (lens[b] > (int64_t)INT32_MAX) return fail(JL_EUNSUPPORTED, "L >= 2^31 (sequence %d)", b);
    if (row0[b] < 0) return fail(JL_EINVAL, "row0 < 0 (sequence %d)", b);
    if (cache_rows >= 0 && row0[b] + lens[b] > cache_rows)
      return fail(JL_EINVAL, "sequence %d: rows %lld + %lld exceed the cache's %lld rows", b, (long long)row0[b],
                  (long long)lens[b], (long long)cache_rows);
    total += lens[b];
  }
  if (dtype != JL_BF16 && dtype != JL_FP32) return fail(JL_EINVAL, "unknown dtype %d", (int)dtype);
  int rc = check_common(w0, w_pretrained, rope_base);
  if (rc) return rc;
  JlHeadMap hm;
  rc = build_head_map(&hm, num_q_heads, num_kv_heads, q_to_kv);
  if (rc) return rc;
  if (dtype != JL_BF16) return fail(JL_EUNSUPPORTED, "decode is built for bf16 caches only");
  if (head_dim != 128) return fail(JL_EUNSUPPORTED, "decode needs head_dim 128");
  if (num_q_heads > 64 || num_kv_heads > 8)
    return fail(JL_EUNSUPPORTED, "decode supports up to 64 q heads and 8 kv heads");
  const int NG = num_q_heads / num_kv_heads;
  if (num_q_heads % num_kv_heads || (NG != 1 && NG != 2 && NG != 4 && NG != 8))
    return fail(JL_EUNSUPPORTED, "decode needs 1, 2, 4 or 8 q heads per kv head");
  {
    int cnt[8] = {0};
    for (int h = 0; h < num_q_heads; ++h) cnt[hm.kv_of[h]]++;
    for (int g = 0; g < num_kv_heads; ++g)
      if (cnt[g] != NG) return fail(JL_EUNSUPPORTED, "decode needs the same number of q heads per kv head");
  }
  if (total > (int64_t)INT32_MAX * 16) return fail(JL_EUNSUPPORTED, "too many keys in one call");
  JlDecSeqs ds;
  jl_decode_plan(lens, row0, num_seqs, w0, w_pretrained, jl_device_shape().cus, &ds);
  const size_t need = total == 0 ? 0 : jl_decode_workspace_bytes(ds, num_q_heads);
  if (workspace == nullptr) {
    *workspace_bytes = need;
    return JL_OK;
  }
  if (*workspace_bytes < need) return fail(JL_ENOSPC, "workspace has %zu bytes, %zu needed", *workspace_bytes, need);
  if (total == 0) return JL_OK;
  if (!q || !k_cache || !v_cache || !o) return fail(JL_EINVAL, "q, caches and o must be device pointers");
  if (((uintptr_t)workspace & 15) || (((uintptr_t)q | (uintptr_t)k_cache | (uintptr_t)v_cache) & 15))
    return fail(JL_EINVAL, "q, caches and workspace must be 16-byte aligned");

  const JlFreqs& fr = freqs_for(head_dim, rope_base);
  const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf((float)head_dim);
  if (g_ev_before) (void)hipEventRecord(g_ev_before, (hipStream_t)hip_stream);
  hipError_t e = jl_launch_decode_bf16(q, k_cache, v_cache, ds, o, lse, num_q_heads, num_kv_heads, hm, scale, fr,
                                       workspace, (hipStream_t)hip_stream);
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  if (g_ev_after) (void)hipEventRecord(g_ev_after, (hipStream_t)hip_stream);
  return JL_OK;
}

JL_EXPORT int jl_bifocal_decode(const void* q, const void* k_cache, const void* v_cache, int64_t L,
                                void* o, float* lse, int32_t num_q_heads, int32_t num_kv_heads,
                                const int32_t* q_to_kv, int32_t head_dim, jl_dtype dtype, int64_t w0,
                                int64_t w_pretrained, double rope_base, float softmax_scale,
                                void* workspace, size_t* workspace_bytes, void* hip_stream) {
  const int64_t row0 = 0;
  return decode_impl(q, k_cache, v_cache, -1, &row0, &L, 1, o, lse, num_q_heads, num_kv_heads, q_to_kv, head_dim,
                     dtype, w0, w_pretrained, rope_base, softmax_scale, workspace, workspace_bytes, hip_stream);
}

JL_EXPORT int jl_bifocal_decode_batch(const void* q, const void* k_cache, const void* v_cache, int64_t cache_rows,
                                      const int64_t* row0, const int64_t* lens, int32_t num_seqs, void* o,
                                      float* lse, int32_t num_q_heads, int32_t num_kv_heads,
                                      const int32_t* q_to_kv, int32_t head_dim, jl_dtype dtype, int64_t w0,
                                      int64_t w_pretrained, double rope_base, float softmax_scale,
                                      void* workspace, size_t* workspace_bytes, void* hip_stream) {
  if (cache_rows < 0) return fail(JL_EINVAL, "cache_rows < 0");
  return decode_impl(q, k_cache, v_cache, cache_rows, row0, lens, num_seqs, o, lse, num_q_heads, num_kv_heads,
                     q_to_kv, head_dim, dtype, w0, w_pretrained, rope_base, softmax_scale, workspace,
                     workspace_bytes, hip_stream);
}

JL_EXPORT int jl_rope_rows(const void* x, void* y, int64_t n_rows, int32_t num_heads, int32_t head_dim,
                           jl_dtype dtype, int64_t pos0, double rope_base, void* hip_stream) {
  if (dtype != JL_BF16 && dtype != JL_FP32) return fail(JL_EINVAL, "unknown dtype %d", (int)dtype);
  if (n_rows < 0) return fail(JL_EINVAL, "n_rows < 0");
  if (pos0 < 0) return fail(JL_EINVAL, "pos0 < 0");
  if (num_heads < 1) return fail(JL_EINVAL, "num_heads must be >= 1");
  if (head_dim < 2 || head_dim % 2 || head_dim / 2 > JL_MAX_HALF)
    return fail(JL_EUNSUPPORTED, "head_dim must be even and <= %d", 2 * JL_MAX_HALF);
  if (!(rope_base > 0.0) || !isfinite(rope_base)) return fail(JL_EINVAL, "rope_base must be finite and > 0");
  if (n_rows > 0 && pos0 + n_rows - 1 > (int64_t)INT32_MAX) return fail(JL_EUNSUPPORTED, "positions >= 2^31");
  if (n_rows == 0) return JL_OK;
  if (!x || !y) return fail(JL_EINVAL, "x and y must be device pointers");
  const JlFreqs& fr = freqs_for(head_dim, rope_base);
  hipError_t e = jl_launch_rope_rows(x, y, dtype == JL_BF16 ? 2 : 4, n_rows, num_heads, head_dim, pos0, fr,
                                     (hipStream_t)hip_stream);
  if (e != hipSuccess) return hip_fail(e, "rope launch");
  return JL_OK;
}

// -------------------------------------------------- decode without allocation

// Split-K partials of jl_bifocal_decode_noalloc.  In host code this name is a
// stand-in, not a device address: kernels get the address that
// hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) char scratch[JL_DECODE_SCRATCH_BYTES];

namespace {
std::once_flag g_scratch_once[JL_MAX_DEVICES];
void* g_scratch_ptr[JL_MAX_DEVICES];
hipError_t g_scratch_err[JL_MAX_DEVICES];

// the scratch's address on the current device, looked up once per device
int scratch_of_current_device(void** ptr) {
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= JL_MAX_DEVICES) return fail(JL_EUNSUPPORTED, "device %d beyond the %d the library serves", dev,
                                                    JL_MAX_DEVICES);
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = p;
  });
  if (g_scratch_err[dev] != hipSuccess) return hip_fail(g_scratch_err[dev], "hipGetSymbolAddress(scratch)");
  *ptr = g_scratch_ptr[dev];
  return JL_OK;
}
}  // namespace

JL_EXPORT int jl_bifocal_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, int64_t L, void* o,
                                        float* lse, int32_t num_q_heads, int32_t num_kv_heads, const int32_t* q_to_kv,
                                        int32_t head_dim, jl_dtype dtype, int64_t w0, int64_t w_pretrained,
                                        double rope_base, float softmax_scale, void* hip_stream) {
  // the size query validates every argument and computes the plan's partials
  size_t need = 0;
  const int64_t row0 = 0;
  int rc = decode_impl(nullptr, nullptr, nullptr, -1, &row0, &L, 1, nullptr, nullptr, num_q_heads, num_kv_heads,
                       q_to_kv, head_dim, dtype, w0, w_pretrained, rope_base, softmax_scale, nullptr, &need, nullptr);
  if (rc) return rc;
  if (need > (size_t)JL_DECODE_SCRATCH_BYTES)
    return fail(JL_EUNSUPPORTED, "this decode needs %zu bytes of partial results; the no-allocation scratch holds %d",
                need, JL_DECODE_SCRATCH_BYTES);
  if (need == 0) return JL_OK;   // L == 0
  if (!q || !k_cache || !v_cache || !o) return fail(JL_EINVAL, "q, caches and o must be device pointers");
  void* ptr = nullptr;
  rc = scratch_of_current_device(&ptr);
  if (rc) return rc;
  size_t cap = JL_DECODE_SCRATCH_BYTES;
  return decode_impl(q, k_cache, v_cache, -1, &row0, &L, 1, o, lse, num_q_heads, num_kv_heads, q_to_kv, head_dim, dtype,
                     w0, w_pretrained, rope_base, softmax_scale, ptr, &cap, hip_stream);
}

// ------------------------------------------------------------------ test hooks

JL_EXPORT int jl_set_profile_events(void* before, void* mid, void* after) {
  if ((before == nullptr) != (after == nullptr)) return fail(JL_EINVAL, "set both events or neither");
  g_ev_before = (hipEvent_t)before;
  g_ev_mid = before == nullptr ? nullptr : (hipEvent_t)mid;
  g_ev_after = (hipEvent_t)after;
  return JL_OK;
}

hipEvent_t jl_profile_mid_event() { return g_ev_mid; }

JL_EXPORT int jl_test_device_shape(int32_t* cus, int32_t* xcds) {
  if (!cus || !xcds) return fail(JL_EINVAL, "bad arguments");
  const JlDevShape s = jl_device_shape();
  *cus = s.cus;
  *xcds = s.xcds;
  return JL_OK;
}

JL_EXPORT int jl_test_decode_plan(const int64_t* lens, int32_t num_seqs, int32_t cus, int32_t* nsub,
                                  int32_t* nwg) {
  if (!lens || !nsub || !nwg || num_seqs < 1 || num_seqs > JL_MAX_SEQS || cus < 1)
    return fail(JL_EINVAL, "bad arguments");
  int64_t row0[JL_MAX_SEQS] = {0};
  for (int b = 0; b < num_seqs; ++b)
    if (lens[b] < 0 || lens[b] > (int64_t)INT32_MAX) return fail(JL_EINVAL, "bad length");
  JlDecSeqs ds;
  jl_decode_plan(lens, row0, num_seqs, 0, 1, cus, &ds);
  *nsub = ds.nsub;
  *nwg = ds.wg_begin[num_seqs];
  return JL_OK;
}

JL_EXPORT int jl_test_decode_prefix(const int64_t* lens, int32_t num_seqs, int32_t cus, int32_t* wg_begin) {
  if (!lens || !wg_begin || num_seqs < 1 || num_seqs > JL_MAX_SEQS || cus < 1)
    return fail(JL_EINVAL, "bad arguments");
  int64_t row0[JL_MAX_SEQS] = {0};
  for (int b = 0; b < num_seqs; ++b)
    if (lens[b] < 0 || lens[b] > (int64_t)INT32_MAX) return fail(JL_EINVAL, "bad length");
  JlDecSeqs ds;
  jl_decode_plan(lens, row0, num_seqs, 0, 1, cus, &ds);
  for (int b = 0; b <= JL_MAX_SEQS; ++b) wg_begin[b] = ds.wg_begin[b];
  return JL_OK;
}

JL_EXPORT int jl_test_group_size_device(const int64_t* L, int64_t n, int64_t w_pretrained, int64_t* G_out,
                                        void* hip_stream) {
  if (n < 0 || w_pretrained < 1 || (n > 0 && (!L || !G_out))) return fail(JL_EINVAL, "bad arguments");
  if (n == 0) return JL_OK;
  hipError_t e = jl_launch_test_group_size(L, n, w_pretrained, G_out, (hipStream_t)hip_stream);
  return e == hipSuccess ? JL_OK : hip_fail(e, "test kernel");
}

JL_EXPORT int jl_test_remote_pos_device(int64_t x0, int64_t n, int64_t G, int32_t* f_out, void* hip_stream) {
  if (x0 < 0 || n < 0 || G < 1 || G > INT32_MAX || x0 + n > (int64_t)INT32_MAX || (n > 0 && !f_out))
    return fail(JL_EINVAL, "bad arguments");
  if (n == 0) return JL_OK;
  hipError_t e = jl_launch_test_remote_pos(x0, n, (int32_t)G, f_out, (hipStream_t)hip_stream);
  return e == hipSuccess ? JL_OK : hip_fail(e, "test kernel");
}

JL_EXPORT int jl_test_rope_angles_device(const int32_t* pos, int64_t n, int32_t m, int32_t head_dim,
                                         double rope_base, float* cos_out, float* sin_out, void* hip_stream) {
  if (n < 0 || head_dim < 2 || head_dim > 2 * JL_MAX_HALF || (head_dim & 1) || m < 0 || m >= head_dim / 2 ||
      !(rope_base > 0.0) || (n > 0 && (!pos || !cos_out || !sin_out)))
    return fail(JL_EINVAL, "bad arguments");
  if (n == 0) return JL_OK;
  const JlFreqs& fr = freqs_for(head_dim, rope_base);
  hipError_t e = jl_launch_test_angles(pos, n, fr.turn_frac[m], cos_out, sin_out, (hipStream_t)hip_stream);
  return e == hipSuccess ? JL_OK : hip_fail(e, "test kernel");
}

JL_EXPORT int jl_bench_mfma_peak(int64_t iters, float* sink, int64_t* flops, void* hip_stream) {
  if (iters < 1 || !sink || !flops) return fail(JL_EINVAL, "bad arguments");
  *flops = (int64_t)jl_device_shape().cus * 8 * iters * 32 * (32 * 32 * 16 * 2);
  hipError_t e = jl_launch_mfma_peak(iters, sink, (hipStream_t)hip_stream);
  return e == hipSuccess ? JL_OK : hip_fail(e, "mfma peak kernel");
}

JL_EXPORT int jl_bench_read_peak(const void* buf, int64_t bytes, int32_t nontemporal, float* sink, void* hip_stream) {
  if (!buf || !sink || bytes < 16 || (bytes & 15) || ((uintptr_t)buf & 15)) return fail(JL_EINVAL, "bad arguments");
  hipError_t e = jl_launch_read_peak(buf, bytes, nontemporal, sink, (hipStream_t)hip_stream);
  return e == hipSuccess ? JL_OK : hip_fail(e, "read peak kernel");
}
