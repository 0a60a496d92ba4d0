// jl_rope.hip - RoPE pre-pass of the prefill path.
//
// Rotates every q and k row once, at its absolute position p (base grid) and
// at its aliased position f(p) = floor(p / G) (remote grid), so the attention
// kernel never re-rotates a key tile per visit (technical summary on
// gist.science, Methodology item 1: classical RoPE inside the local window,
// positions mapped by f beyond it; G per sequence from its length).
// Also writes V transposed for the bf16 attention kernel, whose PV product
// reads 8 consecutive keys of one channel per lane.
#include "jl_internal.h"

int64_t jl_prefill_t_pad(int64_t total_tokens) {
  // a full 128-row q tile and a 64-key tile may start at any row < T
  return ((total_tokens + 128 + 63) / 64) * 64;
}

namespace {

template <typename T>
__device__ inline float ld_f(const T* p) { return (float)(*p); }

template <typename T>
__device__ inline void st_f(T* p, float x) { *p = (T)x; }

// Stores y rounded to T and, when lo != nullptr, the residual y - T(y)
// rounded to T (used for the first positions of a sequence on the bf16 path).
template <typename T>
__device__ inline void st_split(T* hi, T* lo, float y) {
  const T h = (T)y;
  *hi = h;
  if (lo != nullptr) *lo = (T)(y - (float)h);
}

// One thread per (token, frequency m); it rotates pair (m, m + d/2) of every
// q and k head of that token with one sin/cos evaluation per grid.  q is
// multiplied by qscale first.  The bf16 path passes Hq = 0: its prefill
// kernels rotate each query row themselves (scaled by softmax scale *
// log2(e), with the same pair rotation and rounding), so q is never written to
// the workspace; k, its split-operand residuals of the first positions and
// the optional cache output are written here.  With kc set, the
// base-rotated k is also written in the input's [T][Hkv][d] layout: the
// decode cache of the same tokens (technical summary on gist.science,
// Methodology item 2: the cache holds keys rotated at their absolute
// positions), at the cost of one extra write of k instead of a second pass
// over it.
template <typename T>
__global__ void __launch_bounds__(256) rope_prepass_kernel(
    const T* __restrict__ q, const T* __restrict__ k, T* __restrict__ qb, T* __restrict__ qr,
    T* __restrict__ kb, T* __restrict__ kr,
    T* __restrict__ kb_lo, T* __restrict__ kr_lo, T* __restrict__ kc, int64_t total, int64_t t_pad, int Hq,
    int Hkv, int d, JlSeqs seqs, JlFreqs fr, int write_remote, float qscale) {
  const int half = d >> 1;
  const int tpb = 256 / half;               // tokens per block
  const int tl = threadIdx.x / half;
  const int m = threadIdx.x % half;
  const int b = blockIdx.y;
  const int64_t p = (int64_t)blockIdx.x * tpb + tl;

  if (b == seqs.nseq) {                     // zero padding rows T .. t_pad-1
    const int64_t t = total + p;
    if (t >= t_pad) return;
    for (int h = 0; h < Hq; ++h) {
      T* r0 = qb + ((int64_t)h * t_pad + t) * d;
      st_f(r0 + m, 0.f); st_f(r0 + m + half, 0.f);
      if (write_remote) { T* r1 = qr + ((int64_t)h * t_pad + t) * d; st_f(r1 + m, 0.f); st_f(r1 + m + half, 0.f); }
    }
    for (int h = 0; h < Hkv; ++h) {
      T* r0 = kb + ((int64_t)h * t_pad + t) * d;
      st_f(r0 + m, 0.f); st_f(r0 + m + half, 0.f);
      if (write_remote) { T* r1 = kr + ((int64_t)h * t_pad + t) * d; st_f(r1 + m, 0.f); st_f(r1 + m + half, 0.f); }
    }
    return;
  }
  if (p >= seqs.len[b]) {
    // residual rows past the end of a short sequence are zero
    if (kb_lo != nullptr && p < JL_LO_ROWS) {
      const int64_t lrows = (int64_t)seqs.nseq * JL_LO_ROWS;
      const int64_t lrow = (int64_t)b * JL_LO_ROWS + p;
      for (int h = 0; h < Hkv; ++h) {
        st_f(kb_lo + ((int64_t)h * lrows + lrow) * d + m, 0.f);
        st_f(kb_lo + ((int64_t)h * lrows + lrow) * d + m + half, 0.f);
        st_f(kr_lo + ((int64_t)h * lrows + lrow) * d + m, 0.f);
        st_f(kr_lo + ((int64_t)h * lrows + lrow) * d + m + half, 0.f);
      }
    }
    return;
  }
  const int64_t t = seqs.start[b] + p;
  const int pos = (int)p;
  float cb, sb, cr = 1.f, sr = 0.f;
  jl_rope_sincos(pos, fr.turn_frac[m], &sb, &cb);
  if (write_remote) jl_rope_sincos(jl_remote_pos(pos, seqs.G[b]), fr.turn_frac[m], &sr, &cr);

  const bool lo = kb_lo != nullptr && pos < JL_LO_ROWS;
  const int64_t lrow = (int64_t)b * JL_LO_ROWS + pos;
  const int64_t lrows = (int64_t)seqs.nseq * JL_LO_ROWS;
  for (int h = 0; h < Hq; ++h) {
    const T* x = q + (t * Hq + h) * d;
    const float x1 = ld_f(x + m) * qscale, x2 = ld_f(x + m + half) * qscale;
    float y1, y2;
    T* yb = qb + ((int64_t)h * t_pad + t) * d;
    jl_rot_pair(x1, x2, cb, sb, &y1, &y2);
    st_f(yb + m, y1);
    st_f(yb + m + half, y2);
    if (write_remote) {
      T* yr = qr + ((int64_t)h * t_pad + t) * d;
      jl_rot_pair(x1, x2, cr, sr, &y1, &y2);
      st_f(yr + m, y1);
      st_f(yr + m + half, y2);
    }
  }
  for (int h = 0; h < Hkv; ++h) {
    const T* x = k + (t * Hkv + h) * d;
    const float x1 = ld_f(x + m), x2 = ld_f(x + m + half);
    float y1, y2;
    T* yb = kb + ((int64_t)h * t_pad + t) * d;
    T* lb = lo ? kb_lo + ((int64_t)h * lrows + lrow) * d : nullptr;
    jl_rot_pair(x1, x2, cb, sb, &y1, &y2);
    st_split(yb + m, lb ? lb + m : nullptr, y1);
    st_split(yb + m + half, lb ? lb + m + half : nullptr, y2);
    if (kc != nullptr) {
      T* yc = kc + (t * Hkv + h) * d;
      st_f(yc + m, y1);
      st_f(yc + m + half, y2);
    }
    if (write_remote) {
      T* yr = kr + ((int64_t)h * t_pad + t) * d;
      T* lr = lo ? kr_lo + ((int64_t)h * lrows + lrow) * d : nullptr;
      jl_rot_pair(x1, x2, cr, sr, &y1, &y2);
      st_split(yr + m, lr ? lr + m : nullptr, y1);
      st_split(yr + m + half, lr ? lr + m + half : nullptr, y2);
    }
  }
}

// Base RoPE of n consecutive rows x[r][h][:] at positions pos0 + r (one
// thread per (row, m), every head of the row with one sin/cos evaluation):
// the rotation the prefill pre-pass applies on the base grid, for callers
// that build or extend a decode cache of base-rotated keys, or rotate the
// newest query (technical summary on gist.science, Methodology item 2: the
// cache holds keys rotated at their absolute positions).  y may alias x.
// Grid-stride over the n * d/2 (row, m) items, so any row count fits one
// dispatch.
template <typename T>
__global__ void __launch_bounds__(256) rope_rows_kernel(const T* x, T* y, int64_t n, int H, int d,
                                                        int64_t pos0, JlFreqs fr) {
  const int half = d >> 1;
  const int64_t items = n * half;
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < items; e += stride) {
    const int64_t r = e / half;
    const int m = (int)(e - r * half);
    float c, s;
    jl_rope_sincos((int32_t)(pos0 + r), fr.turn_frac[m], &s, &c);
    for (int h = 0; h < H; ++h) {
      const T* xr = x + (r * H + h) * d;
      T* yr = y + (r * H + h) * d;
      const float x1 = ld_f(xr + m), x2 = ld_f(xr + m + half);
      float y1, y2;
      jl_rot_pair(x1, x2, c, s, &y1, &y2);
      st_f(yr + m, y1);
      st_f(yr + m + half, y2);
    }
  }
}

// v [T][Hkv][128] bf16 -> vt [Hkv][vt_cols / 64][128][64] (V^T in 64-key
// tiles), 64 tokens of one sequence per block through LDS; keys past the
// sequence end are zero.
__global__ void __launch_bounds__(256) transpose_v_kernel(const __bf16* __restrict__ v,
                                                          __bf16* __restrict__ vt, int64_t vt_cols,
                                                          int Hkv, JlSeqs seqs) {
  constexpr int D = 128, TB = 64, P = D + 8;
  __shared__ __bf16 tile[TB * P];
  const int h = blockIdx.y, b = blockIdx.z;
  const int p0 = blockIdx.x * TB;
  const int L = seqs.len[b];
  if (p0 >= L) return;
  const int64_t s0 = seqs.start[b];
  const int tid = threadIdx.x;
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int c = it * 256 + tid;
    const int tok = c >> 4, col = (c & 15) * 8;
    uint4 val = make_uint4(0, 0, 0, 0);
    if (p0 + tok < L) val = *(const uint4*)(v + ((s0 + p0 + tok) * Hkv + h) * D + col);
    *(uint4*)(tile + tok * P + col) = val;
  }
  __syncthreads();
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int c = it * 256 + tid;
    const int dd = c >> 3, tk = (c & 7) * 8;
    __bf16 out[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) out[e] = tile[(tk + e) * P + dd];
    // tile-major: 64-key tile n of kv head h is a contiguous [128][64] block
    const int64_t tile = (seqs.vstart[b] + p0) / 64;
    *(uint4*)(vt + (((int64_t)h * (vt_cols / 64) + tile) * D + dd) * 64 + tk) = *(const uint4*)out;
  }
}

}  // namespace

hipError_t jl_launch_rope_prepass(const void* q, const void* k, const JlPrefillWs& ws, int elem_bytes,
                                  int64_t total_tokens, int32_t Hq, int32_t Hkv, int32_t d,
                                  const JlSeqs& seqs, const JlFreqs& fr, float qscale, hipStream_t st) {
  const int half = d / 2;
  const int tpb = 256 / half;
  int32_t max_len = 0;
  for (int b = 0; b < seqs.nseq; ++b) max_len = seqs.len[b] > max_len ? seqs.len[b] : max_len;
  const int64_t pad_rows = ws.t_pad - total_tokens;
  int64_t need = (max_len > pad_rows ? max_len : pad_rows);
  if (ws.kb_lo != nullptr && need < JL_LO_ROWS) need = JL_LO_ROWS;
  dim3 grid((unsigned)((need + tpb - 1) / tpb), (unsigned)(seqs.nseq + 1));
  const int wr = seqs.any_remote;
  if (elem_bytes == 2) {
    rope_prepass_kernel<__bf16><<<grid, 256, 0, st>>>(
        (const __bf16*)q, (const __bf16*)k, (__bf16*)ws.qb, (__bf16*)ws.qr, (__bf16*)ws.kb,
        (__bf16*)ws.kr, (__bf16*)ws.kb_lo,
        (__bf16*)ws.kr_lo, (__bf16*)ws.kc, total_tokens, ws.t_pad, Hq, Hkv, d, seqs, fr, wr, qscale);
  } else {
    rope_prepass_kernel<float><<<grid, 256, 0, st>>>(
        (const float*)q, (const float*)k, (float*)ws.qb, (float*)ws.qr, (float*)ws.kb,
        (float*)ws.kr, nullptr, nullptr, (float*)ws.kc, total_tokens, ws.t_pad, Hq, Hkv,
        d, seqs, fr, wr, qscale);
  }
  return hipGetLastError();
}

hipError_t jl_launch_transpose_v(const void* v, const JlPrefillWs& ws, const JlSeqs& seqs,
                                 int32_t Hkv, hipStream_t st) {
  int32_t max_len = 0;
  for (int b = 0; b < seqs.nseq; ++b) max_len = seqs.len[b] > max_len ? seqs.len[b] : max_len;
  if (max_len == 0) return hipSuccess;
  dim3 grid((unsigned)((max_len + 63) / 64), (unsigned)Hkv, (unsigned)seqs.nseq);
  transpose_v_kernel<<<grid, 256, 0, st>>>((const __bf16*)v, (__bf16*)ws.vt, seqs.vt_cols, Hkv, seqs);
  return hipGetLastError();
}

hipError_t jl_launch_rope_rows(const void* x, void* y, int elem_bytes, int64_t n, int32_t H, int32_t d,
                               int64_t pos0, const JlFreqs& fr, hipStream_t st) {
  const int64_t work = n * (d / 2);
  const int64_t need = (work + 255) / 256;
  const unsigned blocks = (unsigned)(need < (1 << 20) ? need : (1 << 20));   // then grid-stride
  if (elem_bytes == 2)
    rope_rows_kernel<__bf16><<<blocks, 256, 0, st>>>((const __bf16*)x, (__bf16*)y, n, H, d, pos0, fr);
  else
    rope_rows_kernel<float><<<blocks, 256, 0, st>>>((const float*)x, (float*)y, n, H, d, pos0, fr);
  return hipGetLastError();
}
