// jl_decode.hip - bifocal decode against a base-RoPE KV cache, one query
// token for each of one or more sequences.
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
// Split-K: workgroup w covers keys [w C, (w+1) C) of its sequence for every
// head and writes unnormalised partial statistics (max, sum, accumulator) per
// head; a second kernel merges each sequence's partials through their
// LogSumExp values.  Sequences are independent: each has its own length, G,
// cache rows and query, and its own range of workgroups.
//
// A workgroup has one wave per kv head (8 waves) and walks its keys in
// 64-key sub-chunks:
//   angles  the workgroup fills an LDS table of fp32 cos/sin(Delta_j theta_m)
//           for the sub-chunk's remote keys, shared by every kv head.  A thread
//           owns one m and every eighth key: it evaluates the first angle
//           exactly and steps to the next key by composing with one of two
//           fixed rotations (over 8 keys Delta moves by floor(8/G) - 8 or
//           that plus one), one complex product per entry;
//   scores  per 16-key block a lane holds one key's rotary pairs (m, m + 64)
//           for 16 values of m, rotates them in fp32 registers (one bf16
//           rounding, of the rotated key) and feeds them as the A operand of
//           v_mfma_f32_16x16x32_bf16 against the query block (B operand: the
//           kv head's q heads as columns);
//   softmax the sub-chunk's scores of a head sit in 4 lanes x 16 values, so
//           the max and sum need two lane exchanges; the result is online
//           across sub-chunks.  Probabilities go to a wave-private LDS row
//           in bf16, key pairs packed;
//   PV      O^T = V^T P^T on the same MFMA: a lane loads 16 bytes (8
//           channels) of 8 consecutive keys, regroups them with byte
//           permutes into one 8-key operand per channel, and the q heads are
//           the columns again.
// The K and V registers of a sub-chunk are refilled with the next
// sub-chunk's rows as soon as they have been consumed (K per 16-key block
// of the scores, V per 32-key half of PV), so every wave keeps about a
// sub-chunk of loads in flight while it computes, issued a few at a time.
// The angle table has three buffers, filled two sub-chunks ahead; the waves
// synchronise only through per-wave counts of finished sub-chunks in LDS,
// so a wave may run up to a sub-chunk ahead of the slowest one.
#include "jl_internal.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int D = 128;
constexpr int NT = 512;           // one wave per kv head
constexpr int SUB = 64;            // keys per sub-chunk
constexpr int NWAVES = NT / 64;
constexpr int TRIG_STEP = NWAVES;  // key stride of an angle-table thread
constexpr int NTRIG = 3;           // angle-table buffers
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;
constexpr int MAX_HKV = 8;
constexpr int QPITCH = D + 8;      // bf16 elements per query row in LDS
constexpr int TPITCH = 64 + 2;     // float2 entries per angle-table row
constexpr int BUF_RSRC_WORD3 = 0x00020000;   // raw buffer, 32-bit data format
// Cache-policy operands of the tile loads.  Every cache row is read once per
// step.  V rows are loaded non-temporal (nt), K rows with the default policy.
constexpr int K_LOAD_AUX = 0;
constexpr int V_LOAD_AUX = 2;

__device__ inline f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ inline float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ inline uint32_t pack_bf16(float a, float b) {
  const bf16x2 t = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, t);
}

// The lane's index, produced where it is used: addresses built from it are
// not kept in a register across the key loop (they would only be needed
// once per sub-chunk, and the register file is full).
__device__ inline int lane_now() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

// channel held in slot j of MFMA step kb by lane group gq (0..3): the lane
// holds the rotary pairs (16 gq + x, 64 + 16 gq + x), x = 0..15.
__device__ inline int d_of(int kb, int gq, int j) { return (kb >> 1) * 64 + 16 * gq + 8 * (kb & 1) + j; }

// A wave's work is a sequence of units (sub-chunk, kv head of its pair).
// The registers of a unit's K and V tiles are refilled with the next unit's
// rows as soon as they have been consumed (K after the scores, V after PV),
// so every wave keeps one unit of loads in flight while it computes.
struct KTile { u32x4 w[4][4]; };     // [16-key block][MFMA step]: 16 B of one key
struct VTile { u32x4 w[2][8]; };     // [32-key half][key]: 16 B (8 channels) of one key

// Tile loads go through a buffer resource over the workgroup's own key rows
// ([c_begin, min(c_end, L)) of both caches), so rows past L, and the rows of
// the sub-chunk after the last, read as zero without touching memory;
// `row0` is the sub-chunk's first key relative to c_begin and `lane_off` the
// lane's byte offset inside the tile.
__device__ inline void load_k_blk(KTile& t, int blk, __amdgpu_buffer_rsrc_t rk, int row0, int row_bytes,
                                  int lane_off) {
  const int off = (row0 + blk * 16) * row_bytes + lane_off;
  // MFMA steps kb: channels (kb >> 1) * 64 + 8 (kb & 1) + 16 gq .. + 8
  t.w[blk][0] = __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, K_LOAD_AUX);
  t.w[blk][1] = __builtin_amdgcn_raw_buffer_load_b128(rk, off + 16, 0, K_LOAD_AUX);
  t.w[blk][2] = __builtin_amdgcn_raw_buffer_load_b128(rk, off + 128, 0, K_LOAD_AUX);
  t.w[blk][3] = __builtin_amdgcn_raw_buffer_load_b128(rk, off + 144, 0, K_LOAD_AUX);
}

__device__ inline void load_v_half(VTile& t, int kh, __amdgpu_buffer_rsrc_t rv, int row0, int row_bytes,
                                   int lane_off) {
#pragma unroll
  for (int x = 0; x < 8; ++x)
    t.w[kh][x] = __builtin_amdgcn_raw_buffer_load_b128(rv, (row0 + 32 * kh + x) * row_bytes + lane_off, 0, V_LOAD_AUX);
}

// Scores of one 16-key block against the rotated query columns: the lane's
// key rows k[m], k[m + 64] (4 x 16 bytes, pairs 16 gq ..) are rotated by the
// key's table angles in fp32 and fed as MFMA A operands; steps kb = h take
// rotated k[m] and kb = 2 + h rotated k[m + 64] for pairs 8 h .. 8 h + 7.
// The rotation is not done with v_dot2_f32_bf16 on bf16 angle pairs: that
// rounds the coefficients to bf16 before the rotated key is rounded again
// (up to 6e-3 on the outputs of short caches), and costs the same time
// (same-box A/B: within 1% at 32769, 65537 and 131072 keys).
__device__ inline f32x4 remote_block(const u32x4 (&kw)[4], const float2* trow, const __bf16* qcol, int gq) {
  const uint32_t* a = (const uint32_t*)&kw[0];
  const uint32_t* b = (const uint32_t*)&kw[2];
  f32x4 sr = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    u32x4 w1, w2;
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int x2 = 4 * h + x;    // pairs 2 x2 and 2 x2 + 1: (a, b) = (k[m], k[m + 64])
      const float4 t = *(const float4*)&trow[16 * gq + 2 * x2];   // (c, s) of both pairs, fp32
      const float a0 = bf_lo(a[x2]), a1 = bf_hi(a[x2]), b0 = bf_lo(b[x2]), b1 = bf_hi(b[x2]);
      w1[x] = pack_bf16(__builtin_fmaf(a0, t.x, -b0 * t.y), __builtin_fmaf(a1, t.z, -b1 * t.w));   // a c - b s
      w2[x] = pack_bf16(__builtin_fmaf(a0, t.y, b0 * t.x), __builtin_fmaf(a1, t.w, b1 * t.z));    // a s + b c
    }
    const bf16x8 q1 = *(const bf16x8*)(qcol + d_of(h, gq, 0));
    const bf16x8 q2 = *(const bf16x8*)(qcol + d_of(2 + h, gq, 0));
    sr = mfma16(__builtin_bit_cast(bf16x8, w1), q1, sr);
    sr = mfma16(__builtin_bit_cast(bf16x8, w2), q2, sr);
  }
  return sr;
}

// Waits until every wave of the workgroup has finished `target` sub-chunks
// (done[w] counts wave w's; lane w < NWAVES polls entry w).  A per-wave
// count, not one shared total: a total can reach NWAVES * k while fast waves
// are several sub-chunks ahead and slow ones have not finished sub-chunk
// k - 1.  Every wave counts every sub-chunk whatever it computes, so the
// counts always arrive; the bound only keeps a broken invariant from hanging
// the device (the caller then poisons its results).
__device__ inline bool wait_all(const int* done, int target) {
  const int l = lane_now();
  for (int it = 0; it < (1 << 22); ++it) {
    const int v = l < NWAVES ? __hip_atomic_load(&done[l], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP)
                             : target;
    if (__all(v >= target)) return true;
    __builtin_amdgcn_s_sleep(1);
  }
  return false;
}

// Thread (tk, tm)'s part of a sub-chunk's angle table: m = tm, keys tk + 8 r,
// stepping the thread's angle chain (advanced to the next sub-chunk).
__device__ inline void fill_trig(float2 (*tb)[TPITCH], float4* chain, float4 st, int tid, int tm, int tk,
                                 int thr, int dlo_g) {
  const float4 ch = chain[tid];
  float c = ch.x, s = ch.y;
  int rem = __float_as_int(ch.z);
#pragma unroll
  for (int r = 0; r < SUB / TRIG_STEP; ++r) {
    tb[tk + TRIG_STEP * r][tm] = make_float2(c, s);
    const int r8 = rem + TRIG_STEP;
    const bool up = r8 >= thr;
    rem = r8 - (up ? thr : dlo_g);
    const float sc_ = up ? st.z : st.x, ss_ = up ? st.w : st.y;
    const float cn = c * sc_ - s * ss_;
    s = s * sc_ + c * ss_;
    c = cn;
  }
  chain[tid] = make_float4(c, s, __int_as_float(rem), 0.f);
}

// Partial records, laid out for the merge (nwg: workgroups of the call):
//   part_ml [Hq][nwg][2]    (max in log2 units, sum)
//   part_o  [Hq][nwg][128]  unnormalised accumulator
// The leading arguments (14 dwords, the most gfx950 preloads into scalar
// registers at wave launch; the library's build turns preloading on for
// this file) are everything the first loads of a single-sequence call need:
// the caches, the query, and sequence 0's first cache row and length, the
// sub-chunk count, the head counts, the sequence count and G.  A wave then
// issues its first loads without waiting for a kernel-argument load.
template <int NG>
__global__ void __launch_bounds__(NT) decode_split_kernel(
    const __bf16* __restrict__ kc, const __bf16* __restrict__ vc, const __bf16* __restrict__ q,
    int64_t row0_first, int L_first, int nsub, int Hkv, int Hq, int nseq, int G_first,
    float* __restrict__ part_ml, float* __restrict__ part_o, JlHeadMap hm, JlDecSeqs ds, float scale_log2,
    JlFreqs fr) {
  // Row pitches carry 16 bytes of padding: the 16 lanes of an LDS read pass
  // fetch the same columns of different rows, which then fall on distinct
  // banks.
  __shared__ __align__(16) __bf16 qlds[2][MAX_HKV * NG * QPITCH];   // [variant][slot][d]; slot = kvh*NG + n
  // angle table of the sub-chunk: per (key, m) the fp32 pair
  // c, s = cos, sin(Delta_j theta_m)
  __shared__ __align__(16) float2 trig[NTRIG][SUB][TPITCH];   // [sub-chunk % NTRIG]
  __shared__ __align__(16) uint32_t prob[MAX_HKV][NG][SUB / 2];   // wave-private [q head][key pair]
  // per m the two angle-table step rotations, per thread its angle chain
  // (cos, sin, j mod G) at its next key.  Both live in LDS so that no memory
  // load but the tile prefetches sits in the key loop: the load counter is
  // in order, and waiting on anything else would wait on the prefetches too.
  __shared__ float4 steps[64];
  __shared__ float4 chain[NT];
  __shared__ int done[NWAVES];           // sub-chunks finished (angle-table fills included) per wave

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // The workgroup's sequence (uniform).  Sequence 0's first row, length and
  // G come as arguments (its workgroups start at 0); a batch call searches
  // the prefix sums and reads its sequence's fields.
  int b = 0;
  int L = L_first, G = G_first, wg_first = 0;
  int64_t row0 = row0_first;
  if (nseq > 1) {
    // b = how many sequence starts after the first lie at or before this
    // workgroup (the starts never decrease): lane k - 1 compares start k, so
    // the search is one vector load and a ballot instead of one dependent
    // argument load per sequence
    const int k = lane + 1;
    const int start = ds.wg_begin[min(k, JL_MAX_SEQS)];
    b = __builtin_amdgcn_readfirstlane(__popcll(__ballot(k < nseq && (int)blockIdx.x >= start)));
    L = ds.L[b];
    G = ds.G[b];
    wg_first = ds.wg_begin[b];
    row0 = ds.row0[b];
    // resolved inside the branch: a load still pending where the two paths
    // join would be waited for on the single-sequence path as well
    asm volatile("" : "+s"(L), "+s"(G), "+s"(wg_first), "+s"(row0));
  }
  const int w0 = ds.w0[b];                           // first needed after the first loads
  const int nwg = ds.wg_begin[JL_MAX_SEQS];          // the plan repeats the total past the last sequence
  q += (int64_t)b * Hq * D;
  const int i = L - 1;
  const int c_begin = ((int)blockIdx.x - wg_first) * nsub * SUB;
  const int nsc = min(nsub, (L - c_begin + SUB - 1) / SUB);     // sub-chunks holding keys: >= 1

  const int kl = lane & 15, gq = lane >> 4;        // column / row index, lane group
  const int kvh = wave;                              // this wave's kv head
  const bool active = kvh < Hkv;
  const int tm = tid & 63;

  // Loads the prologue's arithmetic needs go out before the tile loads: the
  // vector load counter completes in order, so a load issued after the tiles
  // could only be waited for together with them, and the query rotation and
  // the angle-table set-up would run after the tiles arrive instead of while
  // they stream in.
  //   qrow: query column kl is q head head_of_slot[kvh * NG + kl % NG] (the
  //         query rows sit in LDS by head; columns past NG repeat real heads,
  //         whose results are never stored);
  //   qa, qb: this thread's query elements, channels tm and tm + 64 of heads
  //         wave + 8 r.
  const uint64_t tf = fr.turn_frac[tm];
  const int qrow = (int)hm.head_of_slot[kvh * NG + (kl & (NG - 1))] * QPITCH;
  __bf16 qa[NG], qb[NG];
#pragma unroll
  for (int r = 0; r < NG; ++r) {
    const int h = min(wave + NWAVES * r, Hq - 1);    // unconditional loads: a branch would wait at its end
    qa[r] = q[h * D + tm];
    qb[r] = q[h * D + tm + 64];
  }

  const int row_bytes = Hkv * D * 2;
  // a wave without a kv head gets empty resources: its tile loads (issued
  // like every other wave's, so that no branch sits between the loads and the
  // waits for them) read zeros without touching memory
  const int nrec = active ? min(L - c_begin, nsub * SUB) * row_bytes : 0;
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const char*)kc + (row0 + c_begin) * row_bytes), 0, nrec, BUF_RSRC_WORD3);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const char*)vc + (row0 + c_begin) * row_bytes), 0, nrec, BUF_RSRC_WORD3);
  const int koff = kl * row_bytes + 256 * kvh + 32 * gq;       // key kl, channels 16 gq ..
  const int voff = 8 * gq * row_bytes + 256 * kvh + 16 * kl;   // key 8 gq, channels 8 kl ..
  KTile kt;
  VTile vt;
#pragma unroll
  for (int blk = 0; blk < 4; ++blk) load_k_blk(kt, blk, rk, 0, row_bytes, koff);
  load_v_half(vt, 0, rv, 0, row_bytes, voff);
  load_v_half(vt, 1, rv, 0, row_bytes, voff);
  {
    // the query in both variants: as given (base; bf16 input, so the base
    // scores carry no rounding of q at all) and rotated by Delta_q.  The
    // softmax scale is applied to the fp32 scores (folded into the exp2
    // argument), not to the bf16 query.
    const int dq = jl_remote_pos(i, G) - i;
    float c, s;
    jl_rope_sincos(dq, tf, &s, &c);
    // rows h >= Hq (past the real heads, never read) get a copy of head
    // Hq - 1: no branch, so the loads above stay ahead of the tiles
#pragma unroll
    for (int r = 0; r < NG; ++r) {
      const int h = wave + NWAVES * r;
      const float x1 = (float)qa[r], x2 = (float)qb[r];
      qlds[0][h * QPITCH + tm] = qa[r];
      qlds[0][h * QPITCH + tm + 64] = qb[r];
      qlds[1][h * QPITCH + tm] = (__bf16)(x1 * c - x2 * s);
      qlds[1][h * QPITCH + tm + 64] = (__bf16)(x2 * c + x1 * s);
    }
  }

  // angle-table stepping: thread (tk, tm) owns m = tm and keys tk + 8 r of
  // every sub-chunk.  Over 8 keys Delta = f(j) - j changes by dlo - 8 or
  // dlo - 7, dlo = floor(8 / G): the second when (j mod G) + 8 >= (dlo + 1) G.
  // The first angle is exact; each later one is the previous composed with
  // the step (one complex product, about an fp32 ulp each).
  const int tk = tid >> 6;
  const int dlo = TRIG_STEP / G;
  const int dlo_g = dlo * G, thr = dlo_g + G;
  {
    float4 st;   // (cos, sin) of both steps for m = tm
    jl_rope_sincos(dlo - TRIG_STEP, tf, &st.y, &st.x);
    jl_rope_sincos(dlo - TRIG_STEP + 1, tf, &st.w, &st.z);
    steps[tm] = st;    // every wave writes the same values
    const int j0 = c_begin + tk;
    const int f0 = jl_remote_pos(j0, G);
    float s, c;
    jl_rope_sincos(f0 - j0, tf, &s, &c);
    chain[tid] = make_float4(c, s, __int_as_float(j0 - f0 * G), 0.f);
    if ((i - c_begin) >= w0) {
      fill_trig(trig[0], chain, st, tid, tm, tk, thr, dlo_g);
      if (nsc > 1 && (i - (c_begin + SUB)) >= w0) fill_trig(trig[1], chain, st, tid, tm, tk, thr, dlo_g);
    }
  }

  f32x4 acc[8];                                      // O^T: channel 32 gq + 8 e + c, q head kl
#pragma unroll
  for (int c = 0; c < 8; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  float run_m = -INFINITY, run_l = 0.f;              // column kl (lanes kl + 16 gq)
  if (tid < NWAVES) done[tid] = 0;
  __syncthreads();
  bool in_time = true;

  for (int sc = 0; sc < nsc; ++sc) {
    const int c0 = c_begin + sc * SUB;
    // sub-chunk sc's table was filled in sub-chunk sc - 2 (or before the
    // loop): every wave has finished that
    if (sc >= 2) in_time &= wait_all(done, sc - 1);
    const float2 (*tb)[TPITCH] = trig[sc % NTRIG];
    float alpha = 1.f;
    if (active) {

    // ---------------- scores: 4 blocks of 16 keys ----------------
    // lane holds S^T[key blk*16 + 4 gq + e][column kl] = q.k, unscaled
    f32x4 sco[4];
    {
#pragma unroll
      for (int blk = 0; blk < 4; ++blk) {
        const int kk = blk * 16 + kl;
        const int j = c0 + kk;
        const bool rem = j < L && (i - j) >= w0;
        const bool any_rem = __any(rem);
        const bool any_loc = __any(j < L && !rem);
        f32x4 sr = {}, sl = {};
        if (any_rem) sr = remote_block(kt.w[blk], tb[kk], &qlds[1][qrow], gq);
        if (any_loc) {
#pragma unroll
          for (int kb = 0; kb < 4; ++kb) {
            const bf16x8 bv = *(const bf16x8*)(&qlds[0][qrow + d_of(kb, gq, 0)]);
            sl = mfma16(__builtin_bit_cast(bf16x8, kt.w[blk][kb]), bv, sl);
          }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int jk = c0 + blk * 16 + 4 * gq + e;
          sco[blk][e] = jk >= L ? -INFINITY : (i - jk) >= w0 ? sr[e] : sl[e];
        }
        load_k_blk(kt, blk, rk, (sc + 1) * SUB, row_bytes, koff);
      }
    }

    // ---------------- softmax per column (q head) over the 64 keys ----------------
    float mx = -INFINITY;
#pragma unroll
    for (int blk = 0; blk < 4; ++blk)
#pragma unroll
      for (int e = 0; e < 4; ++e) mx = fmaxf(mx, sco[blk][e]);
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    // scores are raw q.k: the stabiliser is in log2 units (scale * log2 e folded in)
    const float mn = fmaxf(run_m, mx * scale_log2);   // finite: every sub-chunk has a valid key
    alpha = __builtin_amdgcn_exp2f(run_m - mn);
    float sum = 0.f;
#pragma unroll
    for (int blk = 0; blk < 4; ++blk) {
      float pr[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pr[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sco[blk][e], scale_log2, -mn));
        sum += pr[e];
      }
      if (kl < NG)
        {
          const int ln = lane_now();
          *(uint2*)&prob[wave][ln & 15][blk * 8 + 2 * (ln >> 4)] =
              make_uint2(pack_bf16(pr[0], pr[1]), pack_bf16(pr[2], pr[3]));
        }
    }
    sum += __shfl_xor(sum, 16, 64);
    sum += __shfl_xor(sum, 32, 64);
    run_l = run_l * alpha + sum;
    run_m = mn;
    }   // active
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_s_waitcnt(0xc07f);              // lgkmcnt(0): prob rows written

    if (active) {
    // ---------------- PV: O^T += V^T P^T, 32 keys per MFMA ----------------
    // A operand (row kl, keys 8 gq .. 8 gq + 7): channel 8 kl + c of 8 keys;
    // B operand (column kl): probabilities of q head kl for the same keys.
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] *= alpha;
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      const int ln = lane_now();
      const bf16x8 pb = *(const bf16x8*)&prob[wave][ln & (NG - 1)][16 * kh + 4 * (ln >> 4)];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        u32x4 lo, hi;       // channels 8 kl + 2 w and 8 kl + 2 w + 1, keys in pairs
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          lo[u] = __builtin_amdgcn_perm(vt.w[kh][2 * u + 1][w], vt.w[kh][2 * u][w], 0x05040100u);
          hi[u] = __builtin_amdgcn_perm(vt.w[kh][2 * u + 1][w], vt.w[kh][2 * u][w], 0x07060302u);
        }
        acc[2 * w] = mfma16(__builtin_bit_cast(bf16x8, lo), pb, acc[2 * w]);
        acc[2 * w + 1] = mfma16(__builtin_bit_cast(bf16x8, hi), pb, acc[2 * w + 1]);
      }
      // the half's V registers are free: the next sub-chunk's half
      load_v_half(vt, kh, rv, (sc + 1) * SUB, row_bytes, voff);
    }
    }   // active

    // sub-chunk sc + 2's table goes to the buffer of sub-chunk sc - 1, whose
    // readers are done once every wave has finished sub-chunk sc - 1
    if (sc + 2 < nsc && (i - (c0 + 2 * SUB)) >= w0) {
      if (sc >= 1) in_time &= wait_all(done, sc);
      fill_trig(trig[(sc + 2) % NTRIG], chain, steps[tm], tid, tm, tk, thr, dlo_g);
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);              // lgkmcnt(0): table rows written
    if (lane == 0) __hip_atomic_store(&done[wave], sc + 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
  }
  if (!in_time) run_l = NAN;                   // a count that never arrived: fail loudly
  // ---------------- partial records ----------------
  if (!active || kl >= NG) return;
  // output row 4 gq + e of MFMA c is channel 8 (4 gq + e) + c
  float* dst = part_o + ((int64_t)(kvh * NG + kl) * nwg + blockIdx.x) * D + 32 * gq;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    *(float4*)(dst + 8 * e) = make_float4(acc[0][e], acc[1][e], acc[2][e], acc[3][e]);
    *(float4*)(dst + 8 * e + 4) = make_float4(acc[4][e], acc[5][e], acc[6][e], acc[7][e]);
  }
  if (gq == 0)
    *(float2*)(part_ml + ((int64_t)(kvh * NG + kl) * nwg + blockIdx.x) * 2) = make_float2(run_m, run_l);
}

// Merge of the split-K partials through their LogSumExp statistics.
// Workgroup (slot, part) is one wave and produces 16 channels of one head:
// lane (grp, c4) takes partials grp, grp + 16, ... (sixteen loads in flight
// per round, 16 bytes of channels each) with an online max, and the 16
// groups meet through lane exchanges alone (no LDS, no workgroup barrier).
constexpr int RED_GROUPS = 16;
constexpr int RED_DEPTH = 16;

// Leading arguments (preloaded like the split kernel's): the partials, their
// stride (the call's workgroup count) and sequence 0's workgroup count.
__global__ void __launch_bounds__(64) decode_reduce_kernel(const float* __restrict__ part_ml,
                                                           const float* __restrict__ part_o, int stride,
                                                           int nwg_first, JlDecSeqs ds, int Hq, JlHeadMap hm,
                                                           __bf16* __restrict__ o,
                                                           float* __restrict__ lse) {
  const int slot = blockIdx.x, part = blockIdx.y, sq = blockIdx.z, lane = threadIdx.x;
  int w_first = 0, nwg = nwg_first;                  // this sequence's partials
  if (sq > 0) {
    w_first = ds.wg_begin[sq];
    nwg = ds.wg_begin[sq + 1] - w_first;
  }
  if (nwg == 0) return;                               // L = 0: nothing to write
  const int c4 = lane & 3, grp = lane >> 2;
  const float2* ml = (const float2*)part_ml + (int64_t)slot * stride + w_first;
  const float* po = part_o + ((int64_t)slot * stride + w_first) * D + part * 16 + c4 * 4;
  float m = -INFINITY, l = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int wb = grp; wb < nwg; wb += RED_GROUPS * RED_DEPTH) {
    float2 r[RED_DEPTH];
    float4 v[RED_DEPTH];
#pragma unroll
    for (int u = 0; u < RED_DEPTH; ++u) {
      const int w = wb + RED_GROUPS * u;
      r[u] = w < nwg ? ml[w] : make_float2(-INFINITY, 0.f);
      v[u] = w < nwg ? *(const float4*)(po + (int64_t)w * D) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    float mu = m;
#pragma unroll
    for (int u = 0; u < RED_DEPTH; ++u) mu = fmaxf(mu, r[u].x);
    const float sc = __builtin_amdgcn_exp2f(m - mu);     // partial w = grp exists: mu is finite
    l *= sc;
    acc.x *= sc; acc.y *= sc; acc.z *= sc; acc.w *= sc;
#pragma unroll
    for (int u = 0; u < RED_DEPTH; ++u) {
      const float e = __builtin_amdgcn_exp2f(r[u].x - mu);
      l += e * r[u].y;
      acc.x += e * v[u].x; acc.y += e * v[u].y; acc.z += e * v[u].z; acc.w += e * v[u].w;
    }
    m = mu;
  }
  float M = m;                                  // groups without partials hold -inf; group 0 has partial 0
#pragma unroll
  for (int off = 4; off <= 32; off <<= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
  const float wt = __builtin_amdgcn_exp2f(m - M);   // 0 for groups without partials
  l *= wt;
  acc.x *= wt; acc.y *= wt; acc.z *= wt; acc.w *= wt;
#pragma unroll
  for (int off = 4; off <= 32; off <<= 1) {      // the 16 groups (lane bits 2..5)
    l += __shfl_xor(l, off, 64);
    acc.x += __shfl_xor(acc.x, off, 64);
    acc.y += __shfl_xor(acc.y, off, 64);
    acc.z += __shfl_xor(acc.z, off, 64);
    acc.w += __shfl_xor(acc.w, off, 64);
  }
  if (lane < 4) {                                // lane c4 holds channels part * 16 + 4 c4 .. + 3
    const int head = hm.head_of_slot[slot];
    __bf16* dst = o + ((int64_t)sq * Hq + head) * D + part * 16 + 4 * c4;
    dst[0] = (__bf16)(acc.x / l);
    dst[1] = (__bf16)(acc.y / l);
    dst[2] = (__bf16)(acc.z / l);
    dst[3] = (__bf16)(acc.w / l);
    if (lse != nullptr && part == 0 && lane == 0) lse[(int64_t)sq * Hq + head] = (M + __log2f(l)) * LN2;
  }
}

}  // namespace

// One split workgroup fits per compute unit (its LDS use is above half of the
// 160 KB), so a round of the split launch is one workgroup per compute unit.
constexpr int64_t DEC_MAX_NSUB = 1024;   // 65536 keys per workgroup: byte offsets stay in 32 bits

static int64_t decode_wgs(const int64_t* lens, int nseq, int64_t nsub) {
  int64_t w = 0;
  for (int b = 0; b < nseq; ++b) w += (lens[b] + nsub * SUB - 1) / (nsub * SUB);
  return w;
}

// The smallest sub-chunk count per workgroup whose workgroups all fit one
// round on the compute units: a second, partly filled round would cost a
// whole workgroup's time for a few keys.
static int decode_nsub(const int64_t* lens, int nseq, int64_t cus) {
  if (decode_wgs(lens, nseq, DEC_MAX_NSUB) > cus) return (int)DEC_MAX_NSUB;
  int64_t lo = 1, hi = DEC_MAX_NSUB;
  while (lo < hi) {
    const int64_t mid = (lo + hi) / 2;
    if (decode_wgs(lens, nseq, mid) <= cus) hi = mid;
    else lo = mid + 1;
  }
  return (int)lo;
}

void jl_decode_plan(const int64_t* lens, const int64_t* row0, int32_t nseq, int64_t w0, int64_t w_pretrained,
                    int32_t cus, JlDecSeqs* ds) {
  ds->nseq = nseq;
  ds->nsub = decode_nsub(lens, nseq, cus < 1 ? 1 : cus);
  const int64_t chunk = (int64_t)ds->nsub * SUB;
  int wg = 0;
  for (int b = 0; b < JL_MAX_SEQS; ++b) {
    const bool real = b < nseq;
    const int64_t L = real ? lens[b] : 0;
    const int32_t G = (int32_t)jl_group_size_i64(L, w_pretrained);
    ds->wg_begin[b] = wg;
    ds->L[b] = (int32_t)L;
    ds->G[b] = G;
    // With G = 1 the aliased positions are the absolute ones (Delta = 0):
    // every key takes the base path, and the angle table is never built.
    ds->w0[b] = (w0 > L || G == 1) ? (int32_t)L : (int32_t)w0;
    ds->row0[b] = real ? row0[b] : 0;
    wg += (int)((L + chunk - 1) / chunk);
  }
  ds->wg_begin[JL_MAX_SEQS] = wg;
  for (int b = nseq; b <= JL_MAX_SEQS; ++b) ds->wg_begin[b] = wg;
  // Workspace slots: the plan's workgroups, but never fewer than one round
  // (or the sub-chunk count, when that is smaller).  The workgroup count of
  // the plan falls when nsub steps up (32767 keys: 256 workgroups of 2
  // sub-chunks; 32771 keys: 171 of 3), while this bound never decreases as
  // any length grows, so a workspace sized for the longest step of a
  // generation loop serves every shorter one.
  int64_t subs = 0;
  for (int b = 0; b < nseq; ++b) subs += (lens[b] + SUB - 1) / SUB;
  const int64_t floor_wgs = subs < cus ? subs : cus;
  ds->ws_wgs = wg > floor_wgs ? wg : floor_wgs;
}

size_t jl_decode_workspace_bytes(const JlDecSeqs& ds, int32_t Hq) {
  return (size_t)ds.ws_wgs * Hq * (2 + D) * sizeof(float);
}

hipError_t jl_launch_decode_bf16(const void* q, const void* k_cache, const void* v_cache, const JlDecSeqs& ds,
                                 void* o, float* lse, int32_t Hq, int32_t Hkv, const JlHeadMap& hm, float scale,
                                 const JlFreqs& fr, void* workspace, hipStream_t st) {
  const int nwg = ds.wg_begin[ds.nseq];
  if (nwg == 0) return hipSuccess;
  const int NG = Hq / Hkv;
  float* part_ml = (float*)workspace;
  float* part_o = part_ml + (int64_t)nwg * Hq * 2;
  const float sl2 = scale * LOG2E;
#define JL_DEC(NGV)                                                                          \
  decode_split_kernel<NGV><<<nwg, NT, 0, st>>>(                                             \
      (const __bf16*)k_cache, (const __bf16*)v_cache, (const __bf16*)q, ds.row0[0], ds.L[0], ds.nsub, \
      Hkv, Hq, ds.nseq, ds.G[0], part_ml, part_o, hm, ds, sl2, fr)
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
  decode_reduce_kernel<<<dim3(Hq, 8, ds.nseq), 64, 0, st>>>(part_ml, part_o, nwg, ds.wg_begin[1], ds, Hq, hm,
                                                             (__bf16*)o, lse);
  return hipGetLastError();
}
