// jl_prefill_mfma.hip - bf16 MFMA bifocal causal prefill for gfx950.
//
// The routed result is computed as the inclusion-exclusion merge of three
// flash passes combined through their LogSumExp statistics (technical summary
// on gist.science, Methodology item 2: pass 1 local window with base q/k,
// pass 2 full causal with remote q/k, pass 3 local window with remote q/k; no
// boolean mask matrix - masks come from index comparisons):
//     lse_k = m_k + log l_k,  M = max(lse_1, lse_2),  z_k = exp(lse_k - M),
//     out = (z1 o1 + z2 o2 - z3 o3) / (z1 + z2 - z3).
//
// One workgroup = 4 waves = 128 query rows of one head.  The three passes
// run one after another over the same K/V tile pipeline, each with its own
// running max, sum and accumulator (a literal flash pass):
//   pass 2 (remote q/k, causal)   over every key tile up to the diagonal;
//   pass 1 (base q/k, window)     over the tiles within w0 of the rows;
//   after pass 1 the two results are folded into one partial I-E numerator
//   N = z1 o1 + z2 o2 (with z1 l1, z2 l2 kept), freeing a register block;
//   pass 3 (remote q/k, window)   over the window tiles; then
//   out = (N - z3 o3) / (z1 + max(z2 - z3, 0)).
// Exact shortcuts: G = 1 makes passes 1 and 3 identical, so only pass 2 runs;
// w0 >= L makes passes 2 and 3 identical, so only pass 1 runs.
//
// Tile pipeline: K (64 keys x 128) and V^T (128 x 64 keys) tiles are copied
// global -> LDS with global_load_lds_dwordx4 (no register staging) into two
// buffers, so tile t+1 streams in while tile t is multiplied.  Padded LDS
// rows keep the MFMA operand reads free of bank conflicts.
//
// MFMA layout (v_mfma_f32_32x32x16_bf16, one 32-row block per wave):
//   S^T[key][row] = K Q^T: A = K rows from LDS, B = Q rows from registers;
//   each lane owns one query row (lane % 32) and 16 keys per 32-key block, so
//   row max / sum are lane-local plus one exchange with lane ^ 32.
//   O^T[d][row] += V^T P^T: A = V^T from LDS, B = P^T from the S registers.
//   K rows are loaded with bits 2 and 3 of the row index swapped, which makes
//   the 8 P values a lane feeds to one PV MFMA belong to 8 consecutive keys,
//   i.e. one contiguous 16-byte read of a V^T row.
//
// Work order: block n -> (xcd stream n % 8, slot n / 8).  With Hq % 8 == 0
// each stream owns Hq / 8 heads that share kv heads, so the K/V tiles a head
// group streams stay in that XCD's L2; within a stream the (sequence, q tile)
// units come heaviest first (descending q tile index) for load balance.
#include "jl_internal.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int D = 128;
constexpr int BQ = 128;                 // query rows per workgroup
constexpr int BK = 64;                  // keys per tile
constexpr int NT = 256;                 // threads per workgroup
constexpr int KP = 272;                 // LDS pitch of a K row (256 B + 16 B pad)
constexpr int VP = 144;                 // LDS pitch of a V^T row (128 B + 16 B pad)
constexpr int KT_BYTES = BK * KP;       // 17408
constexpr int VT_BYTES = D * VP;        // 18432
constexpr int KT_INSTR = KT_BYTES / 1024;          // 17 KiB pieces
constexpr int VT_INSTR = VT_BYTES / 1024;          // 18 KiB pieces
constexpr int BUF_BYTES = KT_BYTES + VT_BYTES;
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

__device__ inline f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Tile layouts in LDS: K rows at a 272-byte pitch and V^T rows at a 144-byte
// pitch.  The 16-byte pad shifts consecutive rows by 4 (K) or 36 (V^T)
// banks, so the 16 lanes that read one chunk column of 16 rows hit 16
// different bank groups, and every operand address is a per-lane base plus a
// compile-time offset.
//
// global_load_lds_dwordx4 writes lane l's 16 bytes to LDS base + 16 l, one
// contiguous KiB per wave instruction, so piece n of a tile covers LDS bytes
// [n KiB, n KiB + 1 KiB) and each lane fetches the global chunk that belongs
// at its LDS offset.  Lanes that land in a pad re-fetch the row's first
// chunk (the pad is never read).
__device__ inline void issue_tile(char* buf, const char* kg, const char* vg, int64_t vrow_bytes,
                                  int wave, int lane) {
#pragma unroll
  for (int n = wave; n < KT_INSTR; n += 4) {
    const int off = n * 1024 + lane * 16;
    const int r = off / KP, cb = off - r * KP;
    const int c = cb < 256 ? cb : 0;
    __builtin_amdgcn_global_load_lds(kg + r * 256 + c, (lds_void*)(buf + n * 1024), 16, 0, 0);
  }
#pragma unroll
  for (int n = wave; n < VT_INSTR; n += 4) {
    const int off = n * 1024 + lane * 16;
    const int r = off / VP, cb = off - r * VP;
    const int c = cb < 128 ? cb : 0;
    __builtin_amdgcn_global_load_lds(vg + r * vrow_bytes + c,
                                     (lds_void*)(buf + KT_BYTES + n * 1024), 16, 0, 0);
  }
}

__device__ inline void wait_tiles() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

__device__ inline int swap23(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

// S^T for one 64-key tile: s[sb] holds keys sb*32 + 16*(i/8) + 8*g + (i%8)
// of this lane's query row, i = 0..15.
// PRECISE: the operands are split as x = hi + lo (both bf16, lo the rounding
// residual) and S = K_hi Q_hi + K_lo Q_hi + K_hi Q_lo, which keeps about 16
// significant bits of every rotated operand.  Used for the first q tile of a
// sequence: its rows see at most 128 keys, so their LogSumExp is dominated by
// a few scores and does not average out the bf16 rounding of rotated q/k.
template <bool PRECISE>
__device__ inline void score_tile(const char* kt, const bf16x8* qf, const bf16x8* ql,
                                  const __bf16* klo, int lane, f32x16* s) {
  const int g = lane >> 5;
  const int rp = swap23(lane & 31);
#pragma unroll
  for (int sb = 0; sb < 2; ++sb) {
    f32x16 acc = {};
    const int r = sb * 32 + rp;
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) {
      const bf16x8 kh = *(const bf16x8*)(kt + r * KP + kb * 32 + g * 16);
      if constexpr (PRECISE) {
        const bf16x8 kl = *(const bf16x8*)(klo + r * D + kb * 16 + g * 8);
        acc = mfma(kl, qf[kb], acc);
        acc = mfma(kh, ql[kb], acc);
      }
      acc = mfma(kh, qf[kb], acc);
    }
    s[sb] = acc;
  }
}

// o[db] += V^T[db*32 .. +31][keys] * P^T for the 64 keys of the tile.
__device__ inline void pv_tile(const char* vt, const f32x16* p, int lane, f32x16* o) {
  const int g = lane >> 5;
  const int r = lane & 31;
#pragma unroll
  for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      bf16x8 pf;
#pragma unroll
      for (int j = 0; j < 8; ++j) pf[j] = (__bf16)p[sb][8 * hh + j];
      const int c = sb * 4 + hh * 2 + g;
#pragma unroll
      for (int db = 0; db < 4; ++db)
        o[db] = mfma(*(const bf16x8*)(vt + (db * 32 + r) * VP + c * 16), pf, o[db]);
    }
  }
}

// key index (within the tile) of value i of score block sb in a lane of half g
__device__ inline int key_of(int sb, int i, int g) { return sb * 32 + 16 * (i >> 3) + 8 * g + (i & 7); }

struct PassState {
  float m;      // running max (log2 units), identical in lanes l and l ^ 32
  float l;      // this lane's partial sum
};

// One online-softmax step over the tile held in s (raw scores).  `masked`
// selects the index masks: KIND 0 keeps dist >= 0, KIND 1 keeps 0 <= dist < w0.
template <int KIND>
__device__ inline float softmax_tile(f32x16* s, PassState& st, bool masked, int myrow, int j0,
                                     int w0, float sl2, int g) {
  float mx = -INFINITY;
#pragma unroll
  for (int sb = 0; sb < 2; ++sb)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float x = s[sb][i] * sl2;
      if (masked) {
        const int dist = myrow - (j0 + key_of(sb, i, g));
        const bool keep = KIND == 0 ? dist >= 0 : (dist >= 0 && dist < w0);
        x = keep ? x : -INFINITY;
      }
      s[sb][i] = x;
      mx = fmaxf(mx, x);
    }
  mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
  const float mn = fmaxf(st.m, mx);
  const float base = mn == -INFINITY ? 0.f : mn;
  const float alpha = __builtin_amdgcn_exp2f(st.m - base);
  float sum = 0.f;
#pragma unroll
  for (int sb = 0; sb < 2; ++sb)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float p = __builtin_amdgcn_exp2f(s[sb][i] - base);
      s[sb][i] = p;
      sum += p;
    }
  st.l = st.l * alpha + sum;
  st.m = mn;
  return alpha;
}

__device__ inline void load_q(bf16x8* qf, const __bf16* rowp, int g) {
#pragma unroll
  for (int kb = 0; kb < 8; ++kb) qf[kb] = *(const bf16x8*)(rowp + kb * 16 + g * 8);
}

struct TileSrc {
  const char* k;       // K rows of (kv head, sequence), row-major 256 B rows
  const char* v;       // V^T rows of (kv head, sequence start), 128 channels
  int64_t vrow_bytes;  // bytes between V^T rows
  const __bf16* klo;   // residual K rows (PRECISE), row p of the sequence
};

// Per-tile work of a pass for this wave; returns without work when the wave
// sees no key of the tile (causal) or no key inside the window.
template <int KIND, bool PRECISE>
__device__ inline void pass_tile(const char* buf, const TileSrc& src, int j0, const bf16x8* qf,
                                 const bf16x8* ql, PassState& st, f32x16* o, int iw, int myrow,
                                 int w0, float sl2, int lane) {
  if (j0 > iw + 31) return;                                      // all keys after every row
  if (KIND == 1 && j0 + BK - 1 < iw - w0 + 1) return;            // all keys outside the window
  const int g = lane >> 5;
  bool masked = j0 + BK - 1 > iw;                                // some pair has dist < 0
  if (KIND == 1) masked = masked || (j0 < iw + 31 - w0 + 1);     // some pair has dist >= w0
  f32x16 s[2];
  score_tile<PRECISE>(buf, qf, ql, PRECISE ? src.klo + (int64_t)j0 * D : nullptr, lane, s);
  const float a = softmax_tile<KIND>(s, st, masked, myrow, j0, w0, sl2, g);
#pragma unroll
  for (int db = 0; db < 4; ++db) o[db] *= a;
  pv_tile(buf + KT_BYTES, s, lane, o);
}

// A full pass over key tiles [t0, t1) with the double-buffered pipeline.
// Two iterations per loop trip so that each buffer's LDS reads and the DMA
// into the other buffer refer to distinct LDS objects.
template <int KIND, bool PRECISE>
__device__ inline void run_pass(char* buf0, char* buf1, const TileSrc& src, int t0, int t1,
                                const bf16x8* qf, const bf16x8* ql, PassState& st, f32x16* o,
                                int iw, int myrow, int w0, float sl2, int wave, int lane) {
  __syncthreads();                      // every wave is done with both buffers
  if (t0 >= t1) return;
  issue_tile(buf0, src.k + (int64_t)t0 * BK * 256, src.v + (int64_t)t0 * BK * 2, src.vrow_bytes,
             wave, lane);
  for (int t = t0; t < t1; t += 2) {
    wait_tiles();
    __syncthreads();                    // tile t in buf0; buf1 free
    if (t + 1 < t1)
      issue_tile(buf1, src.k + (int64_t)(t + 1) * BK * 256, src.v + (int64_t)(t + 1) * BK * 2,
                 src.vrow_bytes, wave, lane);
    pass_tile<KIND, PRECISE>(buf0, src, t * BK, qf, ql, st, o, iw, myrow, w0, sl2, lane);
    if (t + 1 >= t1) break;
    wait_tiles();
    __syncthreads();                    // tile t+1 in buf1; buf0 free
    if (t + 2 < t1)
      issue_tile(buf0, src.k + (int64_t)(t + 2) * BK * 256, src.v + (int64_t)(t + 2) * BK * 2,
                 src.vrow_bytes, wave, lane);
    pass_tile<KIND, PRECISE>(buf1, src, (t + 1) * BK, qf, ql, st, o, iw, myrow, w0, sl2, lane);
  }
}

// (sequence, q tile) of work unit u: q tiles >= 1 of every sequence, ordered
// by descending tile index (heaviest first), ties by sequence length.
__device__ inline void unit_to_tile(const JlSched& sc, int u, int* seq, int* qt) {
  int k = 0, U = 0;
  for (; k < sc.nlev; ++k) {
    const int next = k + 1 < sc.nlev ? sc.c[k + 1] : 0;
    const int cnt = (sc.c[k] - next) * (k + 1);
    if (u < U + cnt) break;
    U += cnt;
  }
  const int off = u - U;
  *qt = sc.c[k] - off / (k + 1);
  *seq = sc.perm[off % (k + 1)];
}

// PRECISE = true: the first q tile (rows 0 .. 127) of every sequence, with
// split-operand scores.  PRECISE = false: every other q tile.
template <bool PRECISE>
__global__ void __launch_bounds__(NT, 1) prefill_bf16_kernel(
    const __bf16* __restrict__ qb, const __bf16* __restrict__ qr, const __bf16* __restrict__ kb,
    const __bf16* __restrict__ kr, const __bf16* __restrict__ vt, const __bf16* __restrict__ qb_lo,
    const __bf16* __restrict__ qr_lo, const __bf16* __restrict__ kb_lo,
    const __bf16* __restrict__ kr_lo, __bf16* __restrict__ out, float* __restrict__ lse,
    int64_t total, int64_t t_pad, int Hq, JlHeadMap hm, JlSeqs seqs, JlSched sc, int64_t w0_64,
    float sl2) {
  __shared__ __align__(1024) char buf0[BUF_BYTES];
  __shared__ __align__(1024) char buf1[BUF_BYTES];
  int h, b, qt;
  {
    const int n = blockIdx.x;
    if (PRECISE) {
      b = n / Hq;
      h = sc.head_order[n % Hq];
      qt = 0;
    } else if (sc.xcd_heads > 0) {
      const int s = n & 7, slot = n >> 3;
      const int u = slot / sc.xcd_heads;
      h = sc.head_order[s * sc.xcd_heads + slot % sc.xcd_heads];
      if (u >= sc.total_units) return;
      unit_to_tile(sc, u, &b, &qt);
    } else {
      const int u = n / Hq;
      h = sc.head_order[n % Hq];
      unit_to_tile(sc, u, &b, &qt);
    }
  }
  const int L = seqs.len[b];
  const int i0 = qt * BQ;
  if (i0 >= L) return;
  const int tid = threadIdx.x;
  // wave index in a scalar register: the LDS destination of global_load_lds
  // (M0) must be wave-uniform
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, g = lane >> 5;
  const int kvh = hm.kv_of[h];
  const int64_t s0 = seqs.start[b];
  const int G = seqs.G[b];
  const int w0 = w0_64 > (int64_t)L ? L : (int)w0_64;
  const bool only1 = w0 >= L;               // every pair local: pass 1 alone
  const bool only2 = G == 1 && !only1;       // remote grid == base grid: pass 2 alone
  const int iw = i0 + wave * 32;             // first row of this wave
  const int myrow = iw + (lane & 31);
  const int tiles_end = min((i0 + BQ + BK - 1) / BK, (L + BK - 1) / BK);
  const int tw0 = (i0 - w0 + 1) > 0 ? (i0 - w0 + 1) / BK : 0;   // first window tile

  const int64_t lrows = (int64_t)seqs.nseq * JL_LO_ROWS;
  const int64_t lo_base = (int64_t)b * JL_LO_ROWS;
  const int64_t vcols = seqs.vt_cols;
  TileSrc base_src{(const char*)(kb + ((int64_t)kvh * t_pad + s0) * D),
                   (const char*)(vt + (int64_t)kvh * D * vcols + seqs.vstart[b]), vcols * 2,
                   kb_lo + ((int64_t)kvh * lrows + lo_base) * D};
  TileSrc rem_src{(const char*)(kr + ((int64_t)kvh * t_pad + s0) * D), base_src.v, vcols * 2,
                  kr_lo + ((int64_t)kvh * lrows + lo_base) * D};

  bf16x8 qf[8];
  bf16x8 ql[PRECISE ? 8 : 1];
  f32x16 acc[4], keep[4];
  PassState st2{-INFINITY, 0.f}, st1{-INFINITY, 0.f}, st3{-INFINITY, 0.f};
  float out_scale, lse_ref, lse_den;   // final: o = keep * out_scale

  if (only1) {
    // ---- pass 1 alone ----
    load_q(qf, qb + ((int64_t)h * t_pad + s0 + myrow) * D, g);
    if constexpr (PRECISE) load_q(ql, qb_lo + ((int64_t)h * lrows + lo_base + myrow) * D, g);
#pragma unroll
    for (int db = 0; db < 4; ++db) keep[db] = f32x16{};
    run_pass<1, PRECISE>(buf0, buf1, base_src, 0, tiles_end, qf, ql, st1, keep, iw, myrow, w0, sl2,
                         wave, lane);
    const float l1 = st1.l + __shfl_xor(st1.l, 32, 64);
    out_scale = 1.f / l1;
    lse_ref = st1.m;
    lse_den = l1;
  } else {
    // ---- pass 2: remote q/k, causal ----
    load_q(qf, qr + ((int64_t)h * t_pad + s0 + myrow) * D, g);
    if constexpr (PRECISE) load_q(ql, qr_lo + ((int64_t)h * lrows + lo_base + myrow) * D, g);
#pragma unroll
    for (int db = 0; db < 4; ++db) keep[db] = f32x16{};
    run_pass<0, PRECISE>(buf0, buf1, rem_src, 0, tiles_end, qf, ql, st2, keep, iw, myrow, w0, sl2,
                         wave, lane);
    const float l2 = st2.l + __shfl_xor(st2.l, 32, 64);
    if (only2) {
      out_scale = 1.f / l2;
      lse_ref = st2.m;
      lse_den = l2;
    } else {
      // ---- pass 1: base q/k, window ----
      load_q(qf, qb + ((int64_t)h * t_pad + s0 + myrow) * D, g);
      if constexpr (PRECISE) load_q(ql, qb_lo + ((int64_t)h * lrows + lo_base + myrow) * D, g);
#pragma unroll
      for (int db = 0; db < 4; ++db) acc[db] = f32x16{};
      run_pass<1, PRECISE>(buf0, buf1, base_src, tw0, tiles_end, qf, ql, st1, acc, iw, myrow, w0,
                           sl2, wave, lane);
      const float l1 = st1.l + __shfl_xor(st1.l, 32, 64);
      // fold: M = max(lse_1, lse_2); keep = z1 o1 + z2 o2 (unnormalised: e_k A_k)
      const float lam1 = l1 > 0.f ? st1.m + __log2f(l1) : -INFINITY;
      const float lam2 = st2.m + __log2f(l2);
      const float M = fmaxf(lam1, lam2);
      const float e1 = l1 > 0.f ? __builtin_amdgcn_exp2f(st1.m - M) : 0.f;
      const float e2 = __builtin_amdgcn_exp2f(st2.m - M);
#pragma unroll
      for (int db = 0; db < 4; ++db) keep[db] = e1 * acc[db] + e2 * keep[db];
      const float D1 = e1 * l1, D2 = e2 * l2;
      // ---- pass 3: remote q/k, window ----
      load_q(qf, qr + ((int64_t)h * t_pad + s0 + myrow) * D, g);
      if constexpr (PRECISE) load_q(ql, qr_lo + ((int64_t)h * lrows + lo_base + myrow) * D, g);
#pragma unroll
      for (int db = 0; db < 4; ++db) acc[db] = f32x16{};
      run_pass<1, PRECISE>(buf0, buf1, rem_src, tw0, tiles_end, qf, ql, st3, acc, iw, myrow, w0,
                           sl2, wave, lane);
      const float l3 = st3.l + __shfl_xor(st3.l, 32, 64);
      const float e3 = l3 > 0.f ? __builtin_amdgcn_exp2f(st3.m - M) : 0.f;
      const float D3 = e3 * l3;
      // far-pair mass z2 - z3; it is exactly 0 for rows without remote pairs
      // (passes 2 and 3 then run identical arithmetic) and never negative
      const float Z = D1 + fmaxf(D2 - D3, 0.f);
#pragma unroll
      for (int db = 0; db < 4; ++db) keep[db] -= e3 * acc[db];
      out_scale = 1.f / Z;
      lse_ref = M;
      lse_den = Z;
    }
  }

  if (myrow < L) {
    __bf16* orow = out + ((s0 + myrow) * Hq + h) * D;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        bf16x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = (__bf16)(keep[db][4 * q4 + e] * out_scale);
        *(bf16x4*)(orow + db * 32 + 8 * q4 + 4 * g) = w;
      }
    if (lse != nullptr && g == 0) lse[(int64_t)h * total + s0 + myrow] = (lse_ref + __log2f(lse_den)) * LN2;
  }
}

}  // namespace

void jl_build_sched(const JlSeqs& seqs, const JlHeadMap& hm, int Hq, JlSched* sc) {
  // q tiles >= 1 of every sequence, grouped into levels of equal count
  int c[JL_MAX_SEQS], perm[JL_MAX_SEQS], n = 0;
  for (int b = 0; b < seqs.nseq; ++b) {
    const int tiles = (seqs.len[b] + BQ - 1) / BQ;
    if (tiles > 1) {
      c[n] = tiles - 1;
      perm[n] = b;
      ++n;
    }
  }
  for (int i = 1; i < n; ++i)   // insertion sort, descending by tile count
    for (int j = i; j > 0 && c[j] > c[j - 1]; --j) {
      int t = c[j]; c[j] = c[j - 1]; c[j - 1] = t;
      t = perm[j]; perm[j] = perm[j - 1]; perm[j - 1] = t;
    }
  sc->nlev = n;
  sc->total_units = 0;
  for (int k = 0; k < JL_MAX_SEQS; ++k) {
    sc->c[k] = k < n ? c[k] : 0;
    sc->perm[k] = k < n ? perm[k] : 0;
    if (k < n) sc->total_units += c[k];
  }
  // heads grouped by kv head (stable)
  int o = 0;
  for (int kv = 0; kv < JL_MAX_HEADS && o < Hq; ++kv)
    for (int h = 0; h < Hq; ++h)
      if (hm.kv_of[h] == kv) sc->head_order[o++] = (uint8_t)h;
  for (int h = Hq; h < JL_MAX_HEADS; ++h) sc->head_order[h] = 0;
  sc->xcd_heads = (Hq % 8 == 0) ? Hq / 8 : 0;
}

hipError_t jl_launch_prefill_bf16(const JlPrefillWs& ws, void* o, float* lse, int64_t total_tokens,
                                  int32_t Hq, int32_t Hkv, const JlHeadMap& hm, const JlSeqs& seqs,
                                  int64_t w0, float scale, int32_t max_len, hipStream_t st) {
  (void)Hkv;
  (void)max_len;
  JlSched sc;
  jl_build_sched(seqs, hm, Hq, &sc);
  const float sl2 = scale * LOG2E;
  if (sc.total_units > 0) {
    const unsigned nblk = (unsigned)sc.total_units * (unsigned)Hq;   // multiple of 8 when xcd_heads
    prefill_bf16_kernel<false><<<nblk, NT, 0, st>>>(
        (const __bf16*)ws.qb, (const __bf16*)ws.qr, (const __bf16*)ws.kb, (const __bf16*)ws.kr,
        (const __bf16*)ws.vt, (const __bf16*)ws.qb_lo, (const __bf16*)ws.qr_lo,
        (const __bf16*)ws.kb_lo, (const __bf16*)ws.kr_lo, (__bf16*)o, lse, total_tokens, ws.t_pad,
        Hq, hm, seqs, sc, w0, sl2);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  prefill_bf16_kernel<true><<<(unsigned)(seqs.nseq * Hq), NT, 0, st>>>(
      (const __bf16*)ws.qb, (const __bf16*)ws.qr, (const __bf16*)ws.kb, (const __bf16*)ws.kr,
      (const __bf16*)ws.vt, (const __bf16*)ws.qb_lo, (const __bf16*)ws.qr_lo,
      (const __bf16*)ws.kb_lo, (const __bf16*)ws.kr_lo, (__bf16*)o, lse, total_tokens, ws.t_pad, Hq,
      hm, seqs, sc, w0, sl2);
  return hipGetLastError();
}
