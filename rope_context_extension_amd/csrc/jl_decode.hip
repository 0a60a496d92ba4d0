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
// Split-K: workgroup w covers keys [w C, (w+1) C) for every head and writes
// unnormalised partial statistics (max, sum, accumulator) per head; a second
// kernel merges them through their LogSumExp values.
//
// Inside a workgroup (4 waves), per 64-key sub-chunk:
//   angles  the workgroup fills an LDS table of cos/sin(Delta_j theta_m) for
//           the sub-chunk's remote keys (one evaluation per (key, m), shared
//           by every kv head);
//   scores  wave w owns kv heads 2w and 2w+1.  Per 16-key block a lane holds
//           one key's rotary pairs (m, m + 64) for 16 values of m, rotates
//           them in registers and feeds them as the A operand of
//           v_mfma_f32_16x16x32_bf16 against the query block (B operand:
//           the kv head's q heads as columns);
//   softmax the sub-chunk's scores of a head sit in 4 lanes x 16 values, so
//           the max and sum need two lane exchanges; the result is online
//           across sub-chunks;
//   PV      half a wave per kv head: each lane streams 4 channels of the V
//           rows (8 bytes per key) and accumulates the kv head's q heads
//           with probabilities read from a wave-private LDS row.
// The waves of a workgroup only meet at the angle-table barrier.
#include "jl_internal.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int D = 128;
constexpr int NT = 256;
constexpr int SUB = 64;            // keys per sub-chunk
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;
constexpr int MAX_HQ = 64;

__device__ inline f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ inline float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ inline uint32_t pack_bf16(float a, float b) {
  __bf16 t[2] = {(__bf16)a, (__bf16)b};
  return *(const uint32_t*)t;
}

// channel held in slot j of MFMA step kb by lane group gq (0..3): the lane
// holds the rotary pairs (16 gq + x, 64 + 16 gq + x), x = 0..15.
__device__ inline int d_of(int kb, int gq, int j) { return (kb >> 1) * 64 + 16 * gq + 8 * (kb & 1) + j; }

// Partial records, laid out for the merge:
//   part_ml [Hq][nwg][2]    (max in log2 units, sum)
//   part_o  [Hq][nwg][128]  unnormalised accumulator
template <int NG>
__global__ void __launch_bounds__(NT) decode_split_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ kc, const __bf16* __restrict__ vc,
    float* __restrict__ part_ml, float* __restrict__ part_o, int L, int Hq, int Hkv, JlHeadMap hm,
    int w0, int G, int nsub, int nwg, float scale_log2, JlFreqs fr) {
  __shared__ __align__(16) __bf16 qlds[2][MAX_HQ * D];   // [variant][slot][d]; slot = kvh*NG + n
  __shared__ __align__(16) float2 trig[SUB][64];          // cos/sin(Delta_j theta_m) of the sub-chunk
  __shared__ __align__(16) float prob[4][SUB][2 * NG];    // wave-private probabilities [key][slot]
  __shared__ int heads[MAX_HQ];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int i = L - 1;
  const int c_begin = blockIdx.x * nsub * SUB;

  if (tid < Hq) {
    // slot s = kvh * NG + n  <->  the n-th q head (in head order) of kv head kvh
    const int kvh = tid / NG, n = tid % NG;
    int cnt = 0, hh = 0;
    for (int h = 0; h < Hq; ++h)
      if (hm.kv_of[h] == kvh) {
        if (cnt == n) hh = h;
        ++cnt;
      }
    heads[tid] = hh;
  }
  __syncthreads();
  {
    // the query in both variants: as given (base) and rotated by Delta_q
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

  const int kl = lane & 15, gq = lane >> 4;        // score layout: key, rotary group
  const int half = lane >> 5, pc = (lane & 31) * 4; // PV layout: kv head of the pair, 4 channels
  const int kv0 = 2 * wave;                          // this wave's kv heads: kv0, kv0 + 1
  const bool wave_active = kv0 < Hkv;
  const int my_kvh = kv0 + half;
  const bool pv_active = my_kvh < Hkv;
  float acc[NG][4];
#pragma unroll
  for (int n = 0; n < NG; ++n)
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[n][e] = 0.f;
  float run_m[2] = {-INFINITY, -INFINITY};   // per column n < NG of each kv head of the pair
  float run_l[2] = {0.f, 0.f};               // (lanes with kl = n hold head n's values)

  for (int sc = 0; sc < nsub; ++sc) {
    const int c0 = c_begin + sc * SUB;
    if (c0 >= L) break;
    __syncthreads();                           // previous sub-chunk done with trig
    const bool any_remote = (i - c0) >= w0;    // the sub-chunk's first key is the farthest
    if (any_remote) {
      for (int e = tid; e < SUB * 64; e += NT) {
        const int kk = e >> 6, m = e & 63;
        const int j = min(c0 + kk, L - 1);
        float s, c;
        jl_rope_sincos(jl_remote_pos(j, G) - j, fr.turn_frac[m], &s, &c);
        trig[kk][m] = make_float2(c, s);
      }
    }
    __syncthreads();
    if (!wave_active) continue;

    // ---------------- scores: 4 blocks of 16 keys x 2 kv heads ----------------
    f32x4 sco[2][4];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int kvh = min(kv0 + p, Hkv - 1);
#pragma unroll
      for (int blk = 0; blk < 4; ++blk) {
        const int kk = blk * 16 + kl;
        const int j = c0 + kk;
        const int jj = j < L ? j : L - 1;
        const bool rem = j < L && (i - j) >= w0;
        const __bf16* kp = kc + ((int64_t)jj * Hkv + kvh) * D;
        uint4 kw[4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) kw[kb] = *(const uint4*)(kp + d_of(kb, gq, 0));
        const bool any_rem = __any(rem);
        const bool any_loc = __any(j < L && !rem);
        f32x4 sr = {}, sl = {};
        const int ncol = lane & 15;
        if (any_rem) {
          uint32_t w1[8], w2[8];
          const uint32_t* a = (const uint32_t*)&kw[0];
          const uint32_t* b = (const uint32_t*)&kw[2];
#pragma unroll
          for (int x2 = 0; x2 < 8; ++x2) {
            const float4 cs = *(const float4*)&trig[kk][16 * gq + 2 * x2];   // (c, s) of two pairs
            const float a_lo = bf_lo(a[x2]), a_hi = bf_hi(a[x2]);
            const float b_lo = bf_lo(b[x2]), b_hi = bf_hi(b[x2]);
            w1[x2] = pack_bf16(a_lo * cs.x - b_lo * cs.y, a_hi * cs.z - b_hi * cs.w);
            w2[x2] = pack_bf16(b_lo * cs.x + a_lo * cs.y, b_hi * cs.z + a_hi * cs.w);
          }
#pragma unroll
          for (int kb = 0; kb < 4; ++kb) {
            const uint32_t* src = (kb < 2) ? (w1 + 4 * kb) : (w2 + 4 * (kb - 2));
            bf16x8 bv = {};
            if (ncol < NG) bv = *(const bf16x8*)(&qlds[1][(kvh * NG + ncol) * D + d_of(kb, gq, 0)]);
            sr = mfma16(*(const bf16x8*)src, bv, sr);
          }
        }
        if (any_loc) {
#pragma unroll
          for (int kb = 0; kb < 4; ++kb) {
            bf16x8 bv = {};
            if (ncol < NG) bv = *(const bf16x8*)(&qlds[0][(kvh * NG + ncol) * D + d_of(kb, gq, 0)]);
            sl = mfma16(*(const bf16x8*)&kw[kb], bv, sl);
          }
        }
        // lane holds S^T[key blk*16 + 4 gq + e][column kl]
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int jk = c0 + blk * 16 + 4 * gq + e;
          const float v = ((i - jk) >= w0 ? sr[e] : sl[e]) * scale_log2;
          sco[p][blk][e] = jk < L ? v : -INFINITY;
        }
      }
    }
    // ---------------- softmax per column (q head) over the 64 keys ----------------
    // column kl of kv head kv0 + p: lanes kl + 16 gq, values sco[p][0..3][0..3]
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      float mx = -INFINITY;
#pragma unroll
      for (int blk = 0; blk < 4; ++blk)
#pragma unroll
        for (int e = 0; e < 4; ++e) mx = fmaxf(mx, sco[p][blk][e]);
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float mn = fmaxf(run_m[p], mx);         // finite: every sub-chunk has a valid key
      const float alpha = __builtin_amdgcn_exp2f(run_m[p] - mn);
      float sum = 0.f;
#pragma unroll
      for (int blk = 0; blk < 4; ++blk)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float pr = __builtin_amdgcn_exp2f(sco[p][blk][e] - mn);
          sum += pr;
          if (kl < NG) prob[wave][blk * 16 + 4 * gq + e][p * NG + kl] = pr;
        }
      sum += __shfl_xor(sum, 16, 64);
      sum += __shfl_xor(sum, 32, 64);
      run_l[p] = run_l[p] * alpha + sum;
      run_m[p] = mn;
      // rescale the PV accumulators of this kv head's columns: lanes of half p
      // own the accumulators, column n's alpha lives in lane n
#pragma unroll
      for (int n = 0; n < NG; ++n) {
        const float a_n = __shfl(alpha, n, 64);
        if (half == p) {
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[n][e] *= a_n;
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_s_waitcnt(0xc07f);              // lgkmcnt(0): prob rows written
    // ---------------- PV: half-wave per kv head, 4 channels per lane ----------------
    if (pv_active) {
      const int ntok = min(SUB, L - c0);
      const __bf16* vp = vc + ((int64_t)c0 * Hkv + my_kvh) * D + pc;
      const float* pr = &prob[wave][0][half * NG];
      if (ntok == SUB) {
#pragma unroll 16
        for (int t = 0; t < SUB; ++t) {
          const uint2 vw = *(const uint2*)(vp + (int64_t)t * Hkv * D);
          const float v0 = bf_lo(vw.x), v1 = bf_hi(vw.x), v2 = bf_lo(vw.y), v3 = bf_hi(vw.y);
#pragma unroll
          for (int n = 0; n < NG; ++n) {
            const float p = pr[t * 2 * NG + n];
            acc[n][0] += p * v0;
            acc[n][1] += p * v1;
            acc[n][2] += p * v2;
            acc[n][3] += p * v3;
          }
        }
      } else {
        for (int t = 0; t < ntok; ++t) {
          const uint2 vw = *(const uint2*)(vp + (int64_t)t * Hkv * D);
          const float v0 = bf_lo(vw.x), v1 = bf_hi(vw.x), v2 = bf_lo(vw.y), v3 = bf_hi(vw.y);
#pragma unroll
          for (int n = 0; n < NG; ++n) {
            const float p = pr[t * 2 * NG + n];
            acc[n][0] += p * v0;
            acc[n][1] += p * v1;
            acc[n][2] += p * v2;
            acc[n][3] += p * v3;
          }
        }
      }
    }
  }
  // ---------------- partial records ----------------
  if (!wave_active) return;
  if (pv_active) {
#pragma unroll
    for (int n = 0; n < NG; ++n) {
      const int slot = my_kvh * NG + n;
      *(float4*)(part_o + ((int64_t)slot * nwg + blockIdx.x) * D + pc) =
          make_float4(acc[n][0], acc[n][1], acc[n][2], acc[n][3]);
    }
  }
  if (gq == 0 && kl < NG) {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int kvh = kv0 + p;
      if (kvh < Hkv) {
        const int slot = kvh * NG + kl;
        *(float2*)(part_ml + ((int64_t)slot * nwg + blockIdx.x) * 2) = make_float2(run_m[p], run_l[p]);
      }
    }
  }
}

// Merge of the split-K partials through their LogSumExp statistics.
// Workgroup (slot, quarter) produces 32 channels of one head: thread
// (group, c4) reads channels 4 c4 .. 4 c4 + 3 of partials group, group + 32,
// ... with 16-byte loads, four partials in flight, then the 32 groups are
// summed through LDS.
__global__ void __launch_bounds__(256) decode_reduce_kernel(const float* __restrict__ part_ml,
                                                            const float* __restrict__ part_o, int nwg,
                                                            int Hq, int NG, JlHeadMap hm,
                                                            __bf16* __restrict__ o,
                                                            float* __restrict__ lse) {
  __shared__ float red_m[256];
  __shared__ float red_l[32];
  __shared__ float4 red_a[32][8];
  const int slot = blockIdx.x, quarter = blockIdx.y, tid = threadIdx.x;
  const int c4 = tid & 7, grp = tid >> 3;
  const int kvh = slot / NG, n = slot % NG;
  int cnt = 0, head = 0;
  for (int h = 0; h < Hq; ++h)
    if (hm.kv_of[h] == kvh) {
      if (cnt == n) head = h;
      ++cnt;
    }
  const float2* ml = (const float2*)part_ml + (int64_t)slot * nwg;
  float M = -INFINITY;
  for (int w = tid; w < nwg; w += 256) M = fmaxf(M, ml[w].x);
  red_m[tid] = M;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (tid < s) red_m[tid] = fmaxf(red_m[tid], red_m[tid + s]);
    __syncthreads();
  }
  M = red_m[0];
  float l = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  const float* po = part_o + (int64_t)slot * nwg * D + quarter * 32 + c4 * 4;
  int w = grp;
  for (; w + 96 < nwg; w += 128) {
    float2 r[4];
    float4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      r[u] = ml[w + 32 * u];
      v[u] = *(const float4*)(po + (int64_t)(w + 32 * u) * D);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float e = __builtin_amdgcn_exp2f(r[u].x - M);
      l += e * r[u].y;
      acc.x += e * v[u].x; acc.y += e * v[u].y; acc.z += e * v[u].z; acc.w += e * v[u].w;
    }
  }
  for (; w < nwg; w += 32) {
    const float2 r = ml[w];
    const float4 v = *(const float4*)(po + (int64_t)w * D);
    const float e = __builtin_amdgcn_exp2f(r.x - M);
    l += e * r.y;
    acc.x += e * v.x; acc.y += e * v.y; acc.z += e * v.z; acc.w += e * v.w;
  }
  red_a[grp][c4] = acc;
  if (c4 == 0) red_l[grp] = l;
  __syncthreads();
  if (tid < 32) {
    const int cc = tid >> 2, e = tid & 3;   // channel quarter*32 + 4 cc + e
    float A = 0.f, Lt = 0.f;
    for (int g2 = 0; g2 < 32; ++g2) {
      const float4 a = red_a[g2][cc];
      A += e == 0 ? a.x : e == 1 ? a.y : e == 2 ? a.z : a.w;
      Lt += red_l[g2];
    }
    o[head * D + quarter * 32 + tid] = (__bf16)(A / Lt);
    if (lse != nullptr && quarter == 0 && tid == 0) lse[head] = (M + __log2f(Lt)) * LN2;
  }
}

}  // namespace

static int decode_nsub(int64_t L) {
  // about 512 workgroups at long L, at least one 64-key sub-chunk each
  int64_t n = L / (SUB * 512);
  if (n < 1) n = 1;
  if (n > 16) n = 16;
  return (int)n;
}

static int64_t decode_nwg(int64_t L) {
  const int nsub = decode_nsub(L);
  return (L + (int64_t)nsub * SUB - 1) / ((int64_t)nsub * SUB);
}

size_t jl_decode_workspace_bytes(int64_t L, int32_t Hq, int32_t d) {
  (void)d;
  const int64_t nwg = decode_nwg(L);
  return (size_t)(nwg * Hq * (2 + D) * sizeof(float));
}

hipError_t jl_launch_decode_bf16(const void* q, const void* k_cache, const void* v_cache, int64_t L,
                                 void* o, float* lse, int32_t Hq, int32_t Hkv,
                                 const JlHeadMap& hm, int64_t w0, int32_t G, float scale,
                                 const JlFreqs& fr, void* workspace, hipStream_t st) {
  const int nsub = decode_nsub(L);
  const int nwg = (int)decode_nwg(L);
  const int NG = Hq / Hkv;
  const int w0c = w0 > L ? (int)L : (int)w0;
  float* part_ml = (float*)workspace;
  float* part_o = part_ml + (int64_t)nwg * Hq * 2;
  const float sl2 = scale * LOG2E;
#define JL_DEC(NGV)                                                                          \
  decode_split_kernel<NGV><<<nwg, NT, 0, st>>>((const __bf16*)q, (const __bf16*)k_cache,   \
                                               (const __bf16*)v_cache, part_ml, part_o,     \
                                               (int)L, Hq, Hkv, hm, w0c, G, nsub, nwg, sl2, fr)
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
  if (hipEvent_t mid = jl_profile_mid_event()) (void)hipEventRecord(mid, st);
  decode_reduce_kernel<<<dim3(Hq, 4), 256, 0, st>>>(part_ml, part_o, nwg, Hq, NG, hm, (__bf16*)o, lse);
  return hipGetLastError();
}
