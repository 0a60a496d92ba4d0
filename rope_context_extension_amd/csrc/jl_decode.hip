// jl_decode.hip - single-batch bifocal decode against a base-RoPE KV cache.
//
// The cache holds keys rotated at their absolute positions and is never
// written.  For a key at distance >= w0 from the query, the correction
// rotations Delta_q = f(i) - i and Delta_j = f(j) - j move the query and the
// key to their aliased positions in registers (technical summary on
// gist.science, Methodology item 2, "Inference efficiency mechanisms": RoPE
// rotations compose additively, so R(Delta) applied to a base-rotated vector
// gives the vector rotated at the aliased position).  G is recomputed from L
// at every step, so crossing a G boundary needs no cache work.
//
// Split-K: workgroup w covers keys [w*C, (w+1)*C) for every head and writes
// unnormalised partial (max, sum, accumulator) statistics; a second kernel
// merges them through their LogSumExp values.
//
// Inside a workgroup (4 waves), per 64-key sub-chunk:
//   scores  each wave takes 16 keys; every lane owns one key and 16 rotary
//           pairs (m, m + 64), so the Delta rotation is lane-local and its
//           sin/cos are computed once per (key, m) and reused by every kv
//           head.  S^T = K Q^T runs on v_mfma_f32_16x16x32_bf16 with the
//           (rotated) key rows as the A operand.
//   softmax per head over the 64 keys, online across sub-chunks.
//   PV      vector ALU: each lane streams 4 channels of one kv head's V rows
//           and accumulates the heads that share that kv head.
#include "jl_internal.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int D = 128;
constexpr int NT = 256;
constexpr int SUB = 64;          // keys per sub-chunk
constexpr int PS = 132;          // floats per partial record: m, l, pad, pad, acc[128]
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;
constexpr int MAX_HQ = 64;

__device__ inline f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ inline float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// d index held in slot j of MFMA step kb by lane group gq (0..3): the lane
// holds the rotary pairs (16 gq + x, 64 + 16 gq + x), x = 0..15.
__device__ inline int d_of(int kb, int gq, int j) { return (kb >> 1) * 64 + 16 * gq + 8 * (kb & 1) + j; }

template <int NG>
__global__ void __launch_bounds__(NT) decode_split_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ kc, const __bf16* __restrict__ vc,
    float* __restrict__ part, int L, int Hq, int Hkv, JlHeadMap hm, int w0, int G, int nsub,
    float scale_log2, JlFreqs fr) {
  // slot = kvh * NG + n  <->  q head heads[slot]
  __shared__ __align__(16) __bf16 qlds[2][MAX_HQ * D];   // [variant][slot][d]
  __shared__ float slds[SUB * MAX_HQ];                     // [key][slot]
  __shared__ float mrun[MAX_HQ], lrun[MAX_HQ], alpha[MAX_HQ];
  __shared__ int heads[MAX_HQ];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int i = L - 1;
  const int c_begin = blockIdx.x * nsub * SUB;

  if (tid < Hq) {
    // the n-th q head of kv head k, in head order
    int kvh = tid / NG, n = tid % NG, cnt = 0, hh = 0;
    for (int h = 0; h < Hq; ++h)
      if (hm.kv_of[h] == kvh) {
        if (cnt == n) hh = h;
        ++cnt;
      }
    heads[tid] = hh;
    mrun[tid] = -INFINITY;
    lrun[tid] = 0.f;
  }
  __syncthreads();
  // query in both variants: base (as given) and rotated by Delta_q
  {
    const int dq = jl_remote_pos(i, G) - i;
    for (int e = tid; e < Hq * 64; e += NT) {
      const int slot = e >> 6, m = e & 63;
      const __bf16* qr = q + heads[slot] * D;
      const float x1 = (float)qr[m], x2 = (float)qr[m + 64];
      float c, s;
      jl_rope_sincos(dq, fr.turn_frac[m], &s, &c);
      qlds[0][slot * D + m] = qr[m];
      qlds[0][slot * D + m + 64] = qr[m + 64];
      qlds[1][slot * D + m] = (__bf16)(x1 * c - x2 * s);
      qlds[1][slot * D + m + 64] = (__bf16)(x2 * c + x1 * s);
    }
  }
  __syncthreads();

  // PV ownership: (kv head, 4 channels)
  const int pv_kvh = tid >> 5, pv_c = (tid & 31) * 4;
  float acc[NG][4];
#pragma unroll
  for (int n = 0; n < NG; ++n)
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[n][e] = 0.f;

  const int kl = lane & 15, gq = lane >> 4;
  for (int sc = 0; sc < nsub; ++sc) {
    const int c0 = c_begin + sc * SUB;
    if (c0 >= L) break;
    // ---------------- scores ----------------
    const int j = c0 + wave * 16 + kl;                // this lane's key
    const bool valid = j < L;
    const int jj = valid ? j : L - 1;
    const bool rem = valid && (i - j) >= w0;
    const bool any_rem = __any(rem);
    const bool any_loc = __any(valid && !rem);
    float cs[16], sn[16];
    if (any_rem) {
      const int dj = jl_remote_pos(jj, G) - jj;
#pragma unroll
      for (int x = 0; x < 16; ++x) jl_rope_sincos(dj, fr.turn_frac[16 * gq + x], &sn[x], &cs[x]);
    }
    for (int kvh = 0; kvh < Hkv; ++kvh) {
      const __bf16* kp = kc + ((int64_t)jj * Hkv + kvh) * D;
      uint4 kw[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) kw[kb] = *(const uint4*)(kp + d_of(kb, gq, 0));
      f32x4 sr = {}, sl = {};
      const int ncol = lane & 15;                     // B column = slot within kv head
      if (any_rem) {
        // rotate pairs x: first halves in kw[0], kw[1]; second halves in kw[2], kw[3]
        uint32_t w1[8], w2[8];
        const uint32_t* a = (const uint32_t*)&kw[0];
        const uint32_t* b = (const uint32_t*)&kw[2];
#pragma unroll
        for (int x2 = 0; x2 < 8; ++x2) {
          const float a_lo = bf_lo(a[x2]), a_hi = bf_hi(a[x2]);
          const float b_lo = bf_lo(b[x2]), b_hi = bf_hi(b[x2]);
          const int x = 2 * x2;
          const float y1l = a_lo * cs[x] - b_lo * sn[x], y2l = b_lo * cs[x] + a_lo * sn[x];
          const float y1h = a_hi * cs[x + 1] - b_hi * sn[x + 1], y2h = b_hi * cs[x + 1] + a_hi * sn[x + 1];
          __bf16 t1[2] = {(__bf16)y1l, (__bf16)y1h};
          __bf16 t2[2] = {(__bf16)y2l, (__bf16)y2h};
          w1[x2] = *(const uint32_t*)t1;
          w2[x2] = *(const uint32_t*)t2;
        }
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          const uint32_t* src = (kb < 2) ? (w1 + 4 * kb) : (w2 + 4 * (kb - 2));
          bf16x8 av = *(const bf16x8*)src;
          bf16x8 bv = {};
          if (ncol < NG) bv = *(const bf16x8*)(&qlds[1][(kvh * NG + ncol) * D + d_of(kb, gq, 0)]);
          sr = mfma16(av, bv, sr);
        }
      }
      if (any_loc) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          bf16x8 av = *(const bf16x8*)&kw[kb];
          bf16x8 bv = {};
          if (ncol < NG) bv = *(const bf16x8*)(&qlds[0][(kvh * NG + ncol) * D + d_of(kb, gq, 0)]);
          sl = mfma16(av, bv, sl);
        }
      }
      // lane holds S^T[key 4 gq + e][slot ncol]
      if (ncol < NG) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int kk = wave * 16 + 4 * gq + e;
          const int jk = c0 + kk;
          float v;
          if (jk >= L) v = -INFINITY;
          else v = ((i - jk) >= w0 ? sr[e] : sl[e]) * scale_log2;
          slds[kk * MAX_HQ + kvh * NG + ncol] = v;
        }
      }
    }
    __syncthreads();
    // ---------------- softmax (8 threads per slot) ----------------
    for (int base = 0; base < Hq; base += NT / 8) {
      const int slot = base + (tid >> 3);
      const int part8 = tid & 7;
      float mx = -INFINITY;
      if (slot < Hq) {
#pragma unroll
        for (int e = 0; e < 8; ++e) mx = fmaxf(mx, slds[(part8 * 8 + e) * MAX_HQ + slot]);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 1, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 2, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 4, 64));
      float sum = 0.f;
      float mo = 0.f, mn = 0.f;
      if (slot < Hq) {
        mo = mrun[slot];
        mn = fmaxf(mo, mx);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float* ps = &slds[(part8 * 8 + e) * MAX_HQ + slot];
          const float p = __builtin_amdgcn_exp2f(*ps - mn);
          *ps = p;
          sum += p;
        }
      }
      sum += __shfl_xor(sum, 1, 64);
      sum += __shfl_xor(sum, 2, 64);
      sum += __shfl_xor(sum, 4, 64);
      __syncthreads();   // all reads of mrun done before it is updated
      if (slot < Hq && part8 == 0) {
        const float a = __builtin_amdgcn_exp2f(mo - mn);   // mo = -inf on the first sub-chunk
        alpha[slot] = a;
        lrun[slot] = lrun[slot] * a + sum;
        mrun[slot] = mn;
      }
    }
    __syncthreads();
    // ---------------- PV ----------------
    for (int kvh = pv_kvh; kvh < Hkv; kvh += NT / 32) {
      // (for Hkv > 8 a thread would own several kv heads; callers keep Hkv <= 8)
      float a[NG];
#pragma unroll
      for (int n = 0; n < NG; ++n) a[n] = alpha[kvh * NG + n];
#pragma unroll
      for (int n = 0; n < NG; ++n)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[n][e] *= a[n];
      const int ntok = min(SUB, L - c0);
      const __bf16* vp = vc + ((int64_t)c0 * Hkv + kvh) * D + pv_c;
      for (int t = 0; t < ntok; ++t) {
        const uint2 vw = *(const uint2*)(vp + (int64_t)t * Hkv * D);
        const float v0 = bf_lo(vw.x), v1 = bf_hi(vw.x), v2 = bf_lo(vw.y), v3 = bf_hi(vw.y);
        const float* pr = &slds[t * MAX_HQ + kvh * NG];
#pragma unroll
        for (int n = 0; n < NG; ++n) {
          const float p = pr[n];
          acc[n][0] += p * v0;
          acc[n][1] += p * v1;
          acc[n][2] += p * v2;
          acc[n][3] += p * v3;
        }
      }
    }
    __syncthreads();
  }
  // ---------------- partials ----------------
  float* pw = part + (int64_t)blockIdx.x * Hq * PS;
  if (pv_kvh < Hkv) {
#pragma unroll
    for (int n = 0; n < NG; ++n) {
      const int slot = pv_kvh * NG + n;
      *(float4*)(pw + slot * PS + 4 + pv_c) = make_float4(acc[n][0], acc[n][1], acc[n][2], acc[n][3]);
    }
  }
  if (tid < Hq) {
    pw[tid * PS + 0] = mrun[tid];
    pw[tid * PS + 1] = lrun[tid];
  }
}

// Merge of the split-K partials through their LogSumExp statistics.
// Workgroup (slot, quarter): 32 channels of one head slot; its 256 threads
// split the partial records 8 ways and the 32 channels 32 ways.
__global__ void __launch_bounds__(256) decode_reduce_kernel(const float* __restrict__ part, int nwg,
                                                            int Hq, int NG, JlHeadMap hm,
                                                            __bf16* __restrict__ o,
                                                            float* __restrict__ lse) {
  __shared__ float red_m[256];
  __shared__ float red_l[8], red_a[8][32];
  const int slot = blockIdx.x, quarter = blockIdx.y, tid = threadIdx.x;
  const int c = tid & 31, grp = tid >> 5;
  const int d = quarter * 32 + c;
  // head of this slot (same ordering rule as the split kernel)
  const int kvh = slot / NG, n = slot % NG;
  int cnt = 0, head = 0;
  for (int h = 0; h < Hq; ++h)
    if (hm.kv_of[h] == kvh) {
      if (cnt == n) head = h;
      ++cnt;
    }
  float M = -INFINITY;
  for (int w = tid; w < nwg; w += 256) M = fmaxf(M, part[((int64_t)w * Hq + slot) * PS]);
  red_m[tid] = M;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (tid < s) red_m[tid] = fmaxf(red_m[tid], red_m[tid + s]);
    __syncthreads();
  }
  M = red_m[0];
  float l = 0.f, acc = 0.f;
  for (int w = grp; w < nwg; w += 8) {
    const float* r = part + ((int64_t)w * Hq + slot) * PS;
    const float e = __builtin_amdgcn_exp2f(r[0] - M);
    l += e * r[1];
    acc += e * r[4 + d];
  }
  red_a[grp][c] = acc;
  if (c == 0) red_l[grp] = l;
  __syncthreads();
  if (grp == 0) {
    float A = 0.f, Lt = 0.f;
#pragma unroll
    for (int g2 = 0; g2 < 8; ++g2) {
      A += red_a[g2][c];
      Lt += red_l[g2];
    }
    o[head * D + d] = (__bf16)(A / Lt);
    if (lse != nullptr && quarter == 0 && c == 0) lse[head] = (M + __log2f(Lt)) * LN2;
  }
}

}  // namespace

static int decode_nsub(int64_t L) {
  // about 1024 workgroups at long L, never fewer keys than one sub-chunk
  int64_t n = L / (SUB * 1024);
  if (n < 1) n = 1;
  if (n > 8) n = 8;
  return (int)n;
}

size_t jl_decode_workspace_bytes(int64_t L, int32_t Hq, int32_t d) {
  (void)d;
  const int nsub = decode_nsub(L);
  const int64_t nwg = (L + (int64_t)nsub * SUB - 1) / ((int64_t)nsub * SUB);
  return (size_t)(nwg * Hq * PS * sizeof(float));
}

hipError_t jl_launch_decode_bf16(const void* q, const void* k_cache, const void* v_cache, int64_t L,
                                 void* o, float* lse, int32_t Hq, int32_t Hkv,
                                 const JlHeadMap& hm, int64_t w0, int32_t G, float scale,
                                 const JlFreqs& fr, void* workspace, hipStream_t st) {
  const int nsub = decode_nsub(L);
  const int nwg = (int)((L + (int64_t)nsub * SUB - 1) / ((int64_t)nsub * SUB));
  const int NG = Hq / Hkv;
  const int w0c = w0 > L ? (int)L : (int)w0;
  float* part = (float*)workspace;
  const float sl2 = scale * LOG2E;
#define JL_DEC(NGV)                                                                           \
  decode_split_kernel<NGV><<<nwg, NT, 0, st>>>((const __bf16*)q, (const __bf16*)k_cache,    \
                                               (const __bf16*)v_cache, part, (int)L, Hq, Hkv, \
                                               hm, w0c, G, nsub, sl2, fr)
  switch (NG) {
    case 1: JL_DEC(1); break;
    case 2: JL_DEC(2); break;
    case 4: JL_DEC(4); break;
    case 8: JL_DEC(8); break;
    default: return hipErrorInvalidValue;
  }
#undef JL_DEC
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  decode_reduce_kernel<<<dim3(Hq, 4), 256, 0, st>>>(part, nwg, Hq, NG, hm, (__bf16*)o, lse);
  return hipGetLastError();
}
