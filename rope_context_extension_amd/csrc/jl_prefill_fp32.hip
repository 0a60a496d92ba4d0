// jl_prefill_fp32.hip - fp32 vector-ALU bifocal prefill (the exactness path).
//
// Three online-softmax passes over the keys of one query row, each with its
// own (max, sum, output) statistics, merged by inclusion-exclusion through
// their LogSumExp values (technical summary on gist.science, Methodology
// item 2: local window with base q/k, full causal with remote q/k, local
// window with remote q/k; LSE-stabilised merge with no mask matrix):
//   lse_k = m_k + log l_k,  M = max(lse_1, lse_2),  z_k = exp(lse_k - M),
//   o = (z1 o1 + z2 o2 - z3 o3) / (z1 + z2 - z3),  lse = M + log(z1 + z2 - z3).
// One 64-lane workgroup per (row, head, sequence); the lanes split the head
// dimension and reduce each dot product across the wave.
#include "jl_internal.h"

namespace {

struct Pass {
  float m, l;
};

template <int DPT>
__device__ inline void update(Pass& st, float* acc, float s, const float* vj) {
  const float mn = fmaxf(st.m, s);
  const float a = expf(st.m - mn);   // st.m = -inf on the first key: a = 0
  const float p = expf(s - mn);
  st.l = st.l * a + p;
#pragma unroll
  for (int e = 0; e < DPT; ++e) acc[e] = acc[e] * a + p * vj[e];
  st.m = mn;
}

__device__ inline float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

template <int DPT>
__global__ void __launch_bounds__(64) prefill_fp32_kernel(
    const float* __restrict__ qb, const float* __restrict__ qr, const float* __restrict__ kb,
    const float* __restrict__ kr, const float* __restrict__ v, float* __restrict__ o,
    float* __restrict__ lse, int64_t total, int64_t t_pad, int Hq, int Hkv, JlHeadMap hm,
    JlSeqs seqs, int64_t w0, float scale) {
  constexpr int D = DPT * 64;
  const int i = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int L = seqs.len[b];
  if (i >= L) return;
  const int lane = threadIdx.x;
  const int kvh = hm.kv_of[h];
  const int64_t s0 = seqs.start[b];
  const bool g1 = seqs.G[b] == 1;        // remote grid equals base grid
  const bool all_local = w0 >= L;        // every pair inside the window
  // G = 1: passes 1 and 3 are the same computation and cancel exactly, so the
  // result is pass 2.  w0 >= L: passes 2 and 3 cancel, the result is pass 1.
  const bool only1 = all_local;
  const bool only2 = g1 && !all_local;

  float q1[DPT], q2[DPT];
  const float* qbr = qb + ((int64_t)h * t_pad + s0 + i) * D;
  const float* qrr = qr + ((int64_t)h * t_pad + s0 + i) * D;
#pragma unroll
  for (int e = 0; e < DPT; ++e) { q1[e] = qbr[lane + 64 * e]; q2[e] = qrr[lane + 64 * e]; }

  Pass p1{-INFINITY, 0.f}, p2{-INFINITY, 0.f}, p3{-INFINITY, 0.f};
  float a1[DPT] = {}, a2[DPT] = {}, a3[DPT] = {};
  for (int j = 0; j <= i; ++j) {
    const bool local = (int64_t)(i - j) < w0;
    float vj[DPT];
    const float* vr = v + ((s0 + j) * Hkv + kvh) * D;
#pragma unroll
    for (int e = 0; e < DPT; ++e) vj[e] = vr[lane + 64 * e];
    if (!only1) {
      const float* kk = kr + ((int64_t)kvh * t_pad + s0 + j) * D;
      float part = 0.f;
#pragma unroll
      for (int e = 0; e < DPT; ++e) part += q2[e] * kk[lane + 64 * e];
      const float s = scale * wave_sum(part);
      update<DPT>(p2, a2, s, vj);
      if (local && !only2) update<DPT>(p3, a3, s, vj);
    }
    if (local && !only2) {
      const float* kk = kb + ((int64_t)kvh * t_pad + s0 + j) * D;
      float part = 0.f;
#pragma unroll
      for (int e = 0; e < DPT; ++e) part += q1[e] * kk[lane + 64 * e];
      const float s = scale * wave_sum(part);
      update<DPT>(p1, a1, s, vj);
    }
  }

  float out[DPT];
  float lse_row;
  if (only2 || only1) {
    const Pass& p = only1 ? p1 : p2;
    const float* a = only1 ? a1 : a2;
#pragma unroll
    for (int e = 0; e < DPT; ++e) out[e] = a[e] / p.l;
    lse_row = p.m + logf(p.l);
  } else {
    // inclusion-exclusion merge of the three (o_k, lse_k)
    const float lse1 = p1.l > 0.f ? p1.m + logf(p1.l) : -INFINITY;
    const float lse2 = p2.m + logf(p2.l);
    const float lse3 = p3.l > 0.f ? p3.m + logf(p3.l) : -INFINITY;
    const float M = fmaxf(lse1, lse2);
    const float z1 = expf(lse1 - M), z2 = expf(lse2 - M), z3 = expf(lse3 - M);
    float far_w = z2 - z3;                   // mass of the remote-only pairs
    const bool far = far_w > 0.f;
    if (!far) far_w = 0.f;
    const float Z = z1 + far_w;
#pragma unroll
    for (int e = 0; e < DPT; ++e) {
      const float o1 = p1.l > 0.f ? a1[e] / p1.l : 0.f;
      const float o2 = a2[e] / p2.l;
      const float o3 = p3.l > 0.f ? a3[e] / p3.l : 0.f;
      const float num = z1 * o1 + (far ? z2 * o2 - z3 * o3 : 0.f);
      out[e] = num / Z;
    }
    lse_row = M + logf(Z);
  }
  float* orow = o + ((s0 + i) * Hq + h) * D;
#pragma unroll
  for (int e = 0; e < DPT; ++e) orow[lane + 64 * e] = out[e];
  if (lse != nullptr && lane == 0) lse[(int64_t)h * total + s0 + i] = lse_row;
}

}  // namespace

hipError_t jl_launch_prefill_fp32(const JlPrefillWs& ws, const float* v, float* o, float* lse,
                                  int64_t total_tokens, int32_t Hq, int32_t Hkv, int32_t d,
                                  const JlHeadMap& hm, const JlSeqs& seqs, int64_t w0, float scale,
                                  int32_t max_len, hipStream_t st) {
  dim3 grid((unsigned)max_len, (unsigned)Hq, (unsigned)seqs.nseq);
  if (d == 64) {
    prefill_fp32_kernel<1><<<grid, 64, 0, st>>>((const float*)ws.qb, (const float*)ws.qr,
                                                (const float*)ws.kb, (const float*)ws.kr, v, o, lse,
                                                total_tokens, ws.t_pad, Hq, Hkv, hm, seqs, w0, scale);
  } else {
    prefill_fp32_kernel<2><<<grid, 64, 0, st>>>((const float*)ws.qb, (const float*)ws.qr,
                                                (const float*)ws.kb, (const float*)ws.kr, v, o, lse,
                                                total_tokens, ws.t_pad, Hq, Hkv, hm, seqs, w0, scale);
  }
  return hipGetLastError();
}
