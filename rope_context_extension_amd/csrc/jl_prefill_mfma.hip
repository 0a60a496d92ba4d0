// jl_prefill_mfma.hip - bf16 MFMA bifocal causal prefill for gfx950.
//
// The routed result is computed as the inclusion-exclusion merge of three
// flash-style passes combined through their LogSumExp statistics (technical
// summary on gist.science, Methodology item 2: pass 1 local window with base
// q/k, pass 2 full causal with remote q/k, pass 3 local window with remote
// q/k; no boolean mask matrix - masks come from index comparisons):
//     out = (z1 o1 + z2 o2 - z3 o3) / (z1 + z2 - z3).
//
// Work decomposition (one workgroup = 4 waves = 128 query rows of one head):
//   loop A  key tiles that are remote for every row of the workgroup:
//           pass 2 only, no masks.
//   loop B  key tiles near the diagonal ("band"): pass 2 with the causal
//           mask and pass 3 with the window mask.  Passes 2 and 3 share the
//           score tile S = q_r k_r^T and the running max, so pass 3's
//           statistics are pass 2's restricted to window keys.  When loop B
//           ends both passes are complete and their I-E difference
//           (o2 l2 - o3 l3, l2 - l3) is formed once.
//   loop C  the band tiles again with base q/k: pass 1 with its own max.
//   merge   o = (e1 A1 + e2 (A2 - A3)) / (e1 l1 + e2 (l2 - l3)),
//           e_k = exp(m_k - max(m1, m2)), which is the LSE merge above with
//           unnormalised accumulators A_k = o_k l_k.
// Exact shortcuts: G = 1 makes passes 1 and 3 identical (only pass 2 runs);
// w0 >= L makes passes 2 and 3 identical (only pass 1 runs).
//
// MFMA layout (v_mfma_f32_32x32x16_bf16, one 32-row block per wave):
//   S^T[key][row] = K Q^T: A = K rows from LDS, B = Q rows from registers;
//   each lane then owns one query row (lane % 32) and 16 keys per 32-key
//   block, so row max / sum are lane-local plus one exchange with lane ^ 32.
//   O^T[d][row] += V^T P^T: A = V^T from LDS, B = P^T from the S registers.
//   K rows are loaded with bits 2 and 3 of the row index swapped, which makes
//   the 8 P values a lane feeds to one PV MFMA belong to 8 consecutive keys,
//   i.e. to one contiguous 16-byte read of a V^T row.
#include "jl_internal.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int D = 128;
constexpr int BQ = 128;      // query rows per workgroup
constexpr int BK = 64;       // keys per tile
constexpr int NT = 256;      // threads per workgroup
constexpr int KP = D + 8;    // LDS pitch of a K row, bf16 elements (272 B)
constexpr int VP = BK + 8;   // LDS pitch of a V^T row, bf16 elements (144 B)
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

struct __align__(16) Lds {
  __bf16 k[BK * KP];
  __bf16 vt[D * VP];
};

__device__ inline f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ inline void load_k_tile(__bf16* dst, const __bf16* src, int tid) {
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int c = it * NT + tid;
    const int row = c >> 4, col = (c & 15) * 8;
    *(uint4*)(dst + row * KP + col) = *(const uint4*)(src + row * D + col);
  }
}

__device__ inline void load_vt_tile(__bf16* dst, const __bf16* src, int64_t t_pad, int tid) {
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int c = it * NT + tid;
    const int row = c >> 3, col = (c & 7) * 8;
    *(uint4*)(dst + row * VP + col) = *(const uint4*)(src + row * t_pad + col);
  }
}

// S^T for one 64-key tile: s[sb] holds keys sb*32 + 16*(i/8) + 8*g + (i%8)
// of this lane's query row, i = 0..15.
// PRECISE: the operands are split as x = hi + lo (both bf16, lo the rounding
// residual) and S = K_hi Q_hi + K_lo Q_hi + K_hi Q_lo, which keeps about 16
// significant bits of every rotated operand.  Used for the first q tile of a
// sequence: its rows see at most 128 keys, so their LogSumExp is dominated by
// a few scores and does not average out the bf16 rounding of the rotated q/k.
template <bool PRECISE>
__device__ inline void score_tile(const __bf16* lk, const bf16x8* qf, const bf16x8* ql,
                                  const __bf16* klo, int lane, f32x16* s) {
  const int g = lane >> 5;
  const int r = lane & 31;
  const int rp = (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);   // swap bits 2 and 3
#pragma unroll
  for (int sb = 0; sb < 2; ++sb) {
    f32x16 acc = {};
    const __bf16* kr = lk + (sb * 32 + rp) * KP + g * 8;
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) {
      const bf16x8 kh = *(const bf16x8*)(kr + kb * 16);
      if constexpr (PRECISE) {
        const bf16x8 kl = *(const bf16x8*)(klo + (sb * 32 + rp) * D + g * 8 + kb * 16);
        acc = mfma(kl, qf[kb], acc);
        acc = mfma(kh, ql[kb], acc);
      }
      acc = mfma(kh, qf[kb], acc);
    }
    s[sb] = acc;
  }
}

// o[db] += V^T[db*32 .. +31][keys] * P^T for the 64 keys of the tile.
__device__ inline void pv_tile(const __bf16* lvt, const f32x16* p, int lane, f32x16* o) {
  const int g = lane >> 5;
  const int r = lane & 31;
#pragma unroll
  for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      bf16x8 pf;
#pragma unroll
      for (int j = 0; j < 8; ++j) pf[j] = (__bf16)p[sb][8 * hh + j];
      const __bf16* vr = lvt + r * VP + sb * 32 + 16 * hh + 8 * g;
#pragma unroll
      for (int db = 0; db < 4; ++db) o[db] = mfma(*(const bf16x8*)(vr + db * 32 * VP), pf, o[db]);
    }
  }
}

__device__ inline float lane_max(const f32x16* s) {
  float m = -INFINITY;
#pragma unroll
  for (int sb = 0; sb < 2; ++sb)
#pragma unroll
    for (int i = 0; i < 16; ++i) m = fmaxf(m, s[sb][i]);
  return fmaxf(m, __shfl_xor(m, 32, 64));
}

// Online-softmax step on scores already in log2 units with masked entries at
// -inf.  Returns the rescale factor of the previous accumulators and writes
// p = exp2(s - m_new) into s.
__device__ inline float softmax_step(f32x16* s, float& m, float& lsum) {
  const float mn = fmaxf(m, lane_max(s));
  const float base = mn == -INFINITY ? 0.f : mn;
  const float alpha = __builtin_amdgcn_exp2f(m - base);
  float sum = 0.f;
#pragma unroll
  for (int sb = 0; sb < 2; ++sb)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float p = __builtin_amdgcn_exp2f(s[sb][i] - base);
      s[sb][i] = p;
      sum += p;
    }
  lsum = lsum * alpha + sum;
  m = mn;
  return alpha;
}

__device__ inline void scale_acc(f32x16* o, float a) {
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[db][i] *= a;
}

__device__ inline void load_q(bf16x8* qf, const __bf16* rowp, int g) {
#pragma unroll
  for (int kb = 0; kb < 8; ++kb) qf[kb] = *(const bf16x8*)(rowp + kb * 16 + g * 8);
}

// key index (within the tile) of value i of score block sb in a lane of half g
__device__ inline int key_of(int sb, int i, int g) { return sb * 32 + 16 * (i >> 3) + 8 * g + (i & 7); }

// PRECISE = true: the first q tile (rows 0 .. 127) of every sequence, with
// split-operand scores.  PRECISE = false: every other q tile.
template <bool PRECISE>
__global__ void __launch_bounds__(NT) prefill_bf16_kernel(
    const __bf16* __restrict__ qb, const __bf16* __restrict__ qr, const __bf16* __restrict__ kb,
    const __bf16* __restrict__ kr, const __bf16* __restrict__ vt, const __bf16* __restrict__ qb_lo,
    const __bf16* __restrict__ qr_lo, const __bf16* __restrict__ kb_lo,
    const __bf16* __restrict__ kr_lo, __bf16* __restrict__ out, float* __restrict__ lse,
    int64_t total, int64_t t_pad, int Hq, int ntiles_max, JlHeadMap hm, JlSeqs seqs, int64_t w0_64,
    float scale_log2) {
  __shared__ Lds lds;
  const int h = blockIdx.x;
  // longest rows first; q tile 0 belongs to the PRECISE launch
  const int qt = PRECISE ? 0 : ntiles_max - 1 - (int)blockIdx.y;
  const int b = blockIdx.z;
  const int L = seqs.len[b];
  const int i0 = qt * BQ;
  if (i0 >= L) return;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, g = lane >> 5;
  const int kvh = hm.kv_of[h];
  const int64_t s0 = seqs.start[b];
  const int G = seqs.G[b];
  const int w0 = w0_64 > (int64_t)L ? L : (int)w0_64;   // windows beyond L are all of L
  const bool only1 = w0 >= L;                  // every pair local
  const bool only2 = G == 1 && !only1;          // remote grid == base grid
  const int iw = i0 + wave * 32;                // first row of this wave
  const int myrow = iw + (lane & 31);

  const int tiles_end = min((i0 + BQ + BK - 1) / BK, (L + BK - 1) / BK);
  int nfar = (i0 - w0 + 1) > 0 ? (i0 - w0 + 1) / BK : 0;   // loop A tiles
  if (only1) nfar = 0;
  if (nfar > tiles_end) nfar = tiles_end;

  const __bf16* kbh = kb + (int64_t)kvh * t_pad * D + s0 * D;
  const __bf16* krh = kr + (int64_t)kvh * t_pad * D + s0 * D;
  const __bf16* vth = vt + (int64_t)kvh * D * t_pad + s0;
  // residual rows (PRECISE only): row b * JL_LO_ROWS + p
  const int64_t lrows = (int64_t)seqs.nseq * JL_LO_ROWS;
  const __bf16* kb_loh = kb_lo + ((int64_t)kvh * lrows + (int64_t)b * JL_LO_ROWS) * D;
  const __bf16* kr_loh = kr_lo + ((int64_t)kvh * lrows + (int64_t)b * JL_LO_ROWS) * D;

  f32x16 s[2];
  f32x16 o2[4] = {}, o3[4] = {};
  float m2 = -INFINITY, l2 = 0.f, l3 = 0.f;
  bf16x8 qf[8];
  bf16x8 ql[PRECISE ? 8 : 1];

  if (!only1) {
    load_q(qf, qr + ((int64_t)h * t_pad + s0 + myrow) * D, g);
    if constexpr (PRECISE) load_q(ql, qr_lo + ((int64_t)h * lrows + (int64_t)b * JL_LO_ROWS + myrow) * D, g);
    // ---- loop A: remote-only tiles, pass 2 ----
    for (int t = 0; t < nfar; ++t) {
      __syncthreads();
      load_k_tile(lds.k, krh + (int64_t)t * BK * D, tid);
      load_vt_tile(lds.vt, vth + t * BK, t_pad, tid);
      __syncthreads();
      score_tile<false>(lds.k, qf, ql, nullptr, lane, s);
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) s[sb] *= scale_log2;
      const float a = softmax_step(s, m2, l2);
      scale_acc(o2, a);
      pv_tile(lds.vt, s, lane, o2);
    }
    // ---- loop B: band tiles, pass 2 (causal) and pass 3 (window) ----
    for (int t = nfar; t < tiles_end; ++t) {
      const int j0 = t * BK;
      __syncthreads();
      load_k_tile(lds.k, krh + (int64_t)j0 * D, tid);
      load_vt_tile(lds.vt, vth + j0, t_pad, tid);
      __syncthreads();
      if (j0 > iw + 31) continue;                       // wave sees none of these keys
      const bool any_window = !only2 && (j0 + BK - 1 >= iw - w0 + 1);
      score_tile<PRECISE>(lds.k, qf, ql, kr_loh + (int64_t)j0 * D, lane, s);
      f32x16 s3[2];
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int dist = myrow - (j0 + key_of(sb, i, g));
          const float x = s[sb][i] * scale_log2;
          s[sb][i] = dist >= 0 ? x : -INFINITY;
        }
      const float a = softmax_step(s, m2, l2);
      scale_acc(o2, a);
      if (any_window) {
        float sum3 = 0.f;
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int dist = myrow - (j0 + key_of(sb, i, g));
            const float p = dist < w0 ? s[sb][i] : 0.f;   // p is already 0 where dist < 0
            s3[sb][i] = p;
            sum3 += p;
          }
        l3 = l3 * a + sum3;
        scale_acc(o3, a);
        pv_tile(lds.vt, s3, lane, o3);
      } else if (!only2) {
        l3 *= a;
        scale_acc(o3, a);
      }
      pv_tile(lds.vt, s, lane, o2);
    }
    // I-E difference of passes 2 and 3 (same running max m2)
    if (!only2) {
#pragma unroll
      for (int db = 0; db < 4; ++db) o2[db] -= o3[db];
      l2 -= l3;
    }
  }

  f32x16 o1[4] = {};
  float m1 = -INFINITY, l1 = 0.f;
  if (!only2) {
    load_q(qf, qb + ((int64_t)h * t_pad + s0 + myrow) * D, g);
    if constexpr (PRECISE) load_q(ql, qb_lo + ((int64_t)h * lrows + (int64_t)b * JL_LO_ROWS + myrow) * D, g);
    // ---- loop C: band tiles, pass 1 (window, base q/k) ----
    int tc0 = (i0 - w0 + 1) > 0 ? (i0 - w0 + 1) / BK : 0;
    if (only1) tc0 = 0;
    for (int t = tc0; t < tiles_end; ++t) {
      const int j0 = t * BK;
      __syncthreads();
      load_k_tile(lds.k, kbh + (int64_t)j0 * D, tid);
      load_vt_tile(lds.vt, vth + j0, t_pad, tid);
      __syncthreads();
      if (j0 > iw + 31) continue;
      if (j0 + BK - 1 < iw - w0 + 1) continue;        // no window pair in this wave
      score_tile<PRECISE>(lds.k, qf, ql, kb_loh + (int64_t)j0 * D, lane, s);
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int dist = myrow - (j0 + key_of(sb, i, g));
          const float x = s[sb][i] * scale_log2;
          s[sb][i] = (dist >= 0 && dist < w0) ? x : -INFINITY;
        }
      const float a = softmax_step(s, m1, l1);
      scale_acc(o1, a);
      pv_tile(lds.vt, s, lane, o1);
    }
  }

  // ---- merge ----
  l1 += __shfl_xor(l1, 32, 64);
  l2 += __shfl_xor(l2, 32, 64);
  float e1 = 0.f, e2 = 0.f;
  if (only2) {
    e2 = 1.f;
  } else if (only1) {
    e1 = 1.f;
  } else {
    const bool has1 = l1 > 0.f;
    const bool has2 = l2 > 0.f;                 // remote-only mass survives the difference
    const float mm = fmaxf(has1 ? m1 : -INFINITY, has2 ? m2 : -INFINITY);
    e1 = has1 ? __builtin_amdgcn_exp2f(m1 - mm) : 0.f;
    e2 = has2 ? __builtin_amdgcn_exp2f(m2 - mm) : 0.f;
  }
  const float Z = e1 * l1 + e2 * l2;
  const float inv = 1.f / Z;
  const float c1 = e1 * inv, c2 = e2 * inv;
  if (myrow < L) {
    __bf16* orow = out + ((s0 + myrow) * Hq + h) * D;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        bf16x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 4 * q4 + e;
          w[e] = (__bf16)(c1 * o1[db][i] + c2 * o2[db][i]);
        }
        *(bf16x4*)(orow + db * 32 + 8 * q4 + 4 * g) = w;
      }
    if (lse != nullptr && g == 0) {
      float mref;
      if (only2) mref = m2;
      else if (only1) mref = m1;
      else mref = fmaxf(l1 > 0.f ? m1 : -INFINITY, l2 > 0.f ? m2 : -INFINITY);
      lse[(int64_t)h * total + s0 + myrow] = (mref + __log2f(Z)) * LN2;
    }
  }
}

}  // namespace

hipError_t jl_launch_prefill_bf16(const JlPrefillWs& ws, void* o, float* lse, int64_t total_tokens,
                                  int32_t Hq, int32_t Hkv, const JlHeadMap& hm, const JlSeqs& seqs,
                                  int64_t w0, float scale, int32_t max_len, hipStream_t st) {
  (void)Hkv;
  const int ntiles = (max_len + BQ - 1) / BQ;
  if (ntiles > 1) {
    dim3 grid((unsigned)Hq, (unsigned)(ntiles - 1), (unsigned)seqs.nseq);
    prefill_bf16_kernel<false><<<grid, NT, 0, st>>>(
        (const __bf16*)ws.qb, (const __bf16*)ws.qr, (const __bf16*)ws.kb, (const __bf16*)ws.kr,
        (const __bf16*)ws.vt, (const __bf16*)ws.qb_lo, (const __bf16*)ws.qr_lo,
        (const __bf16*)ws.kb_lo, (const __bf16*)ws.kr_lo, (__bf16*)o, lse, total_tokens, ws.t_pad,
        Hq, ntiles, hm, seqs, w0, scale * LOG2E);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  dim3 grid0((unsigned)Hq, 1u, (unsigned)seqs.nseq);
  prefill_bf16_kernel<true><<<grid0, NT, 0, st>>>(
      (const __bf16*)ws.qb, (const __bf16*)ws.qr, (const __bf16*)ws.kb, (const __bf16*)ws.kr,
      (const __bf16*)ws.vt, (const __bf16*)ws.qb_lo, (const __bf16*)ws.qr_lo,
      (const __bf16*)ws.kb_lo, (const __bf16*)ws.kr_lo, (__bf16*)o, lse, total_tokens, ws.t_pad, Hq,
      ntiles, hm, seqs, w0, scale * LOG2E);
  return hipGetLastError();
}
