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
// Rows from 128 on (prefill_pp_kernel, 256 rows and 8 waves per workgroup):
// one workgroup runs all three passes of its tile.  Pass 1 first; then
// passes 2 and 3 come from one walk over the remote-grid key tiles, window
// tiles first: the walk's state after the window tiles is pass 3's, its end
// state pass 2's, and the far part z2 o2 - z3 o3 is formed from the two
// states and added to pass 1's share in the same workgroup.
//
// A sequence's first 128 rows (prefill_pass_kernel, one workgroup = 4 waves
// = 128 query rows of one head): the three passes run one after another over
// the same K/V tile pipeline, each with its own running max, sum and
// accumulator (a literal flash pass):
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
// Work order: block n -> (xcd stream n % X, slot n / X) for the X XCDs of the
// device (the dispatcher deals workgroups to the XCDs round robin).  With
// Hq % X == 0 each stream owns Hq / X heads that share kv heads, so the K/V tiles a head
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
constexpr int KT_PIECES = KT_BYTES / 1024;          // 17 KiB pieces of a K tile
constexpr int VT_PIECES = VT_BYTES / 1024;          // 18 KiB pieces of a V^T tile
constexpr int K_PER_WAVE = (KT_PIECES + 3) / 4;     // 5
constexpr int V_PER_WAVE = (VT_PIECES + 3) / 4;     // 5
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
// chunk (the pad is never read).  Every wave issues the same number of
// pieces per tile (a wave that runs out repeats its last piece, rewriting
// identical bytes), so waits are the same in every wave.  The per-lane source
// offsets depend only on (wave, lane) and are computed once.
struct DmaPlan {
  uint32_t koff[K_PER_WAVE];   // byte offset of this lane's source chunk in a K tile
  uint32_t voff[V_PER_WAVE];   // ... in a V^T tile
};

__device__ inline DmaPlan make_dma_plan(int wave, int lane) {
  DmaPlan p;
#pragma unroll
  for (int i = 0; i < K_PER_WAVE; ++i) {
    const int n = min(wave + 4 * i, KT_PIECES - 1);
    const int off = n * 1024 + lane * 16;
    const int r = off / KP, cb = off - r * KP;
    p.koff[i] = (uint32_t)(r * 256 + (cb < 256 ? cb : 0));
  }
#pragma unroll
  for (int i = 0; i < V_PER_WAVE; ++i) {
    const int n = min(wave + 4 * i, VT_PIECES - 1);
    const int off = n * 1024 + lane * 16;
    const int r = off / VP, cb = off - r * VP;
    p.voff[i] = (uint32_t)(r * 128 + (cb < 128 ? cb : 0));
  }
  return p;
}

// kg / vg: the tile's first byte in global memory (K rows / V^T block)
__device__ inline void issue_k(char* kbuf, const char* kg, const DmaPlan& p, int wave) {
#pragma unroll
  for (int i = 0; i < K_PER_WAVE; ++i) {
    const int n = min(wave + 4 * i, KT_PIECES - 1);
    __builtin_amdgcn_global_load_lds(kg + p.koff[i], (lds_void*)(kbuf + n * 1024), 16, 0, 0);
  }
}

__device__ inline void issue_v(char* vbuf, const char* vg, const DmaPlan& p, int wave) {
#pragma unroll
  for (int i = 0; i < V_PER_WAVE; ++i) {
    const int n = min(wave + 4 * i, VT_PIECES - 1);
    __builtin_amdgcn_global_load_lds(vg + p.voff[i], (lds_void*)(vbuf + n * 1024), 16, 0, 0);
  }
}

__device__ inline void wait_all_tiles() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

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
  float m;      // stabiliser (log2 units), identical in lanes l and l ^ 32
  float l;      // this lane's partial sum of exp2(s - m)
};

// The stabiliser m of a row is raised only when the row's score maximum
// exceeds it by more than RESCALE_LOG2 (log2 units), so most tiles skip the
// rescale of the accumulators.  Any m works in exact arithmetic (the merge
// uses lse = m + log2 l); the bound keeps every p = exp2(s - m) <= 2^8.
constexpr float RESCALE_LOG2 = 8.f;

// Index masks of a tile: KIND 0 keeps dist >= 0 (causal), KIND 1 keeps
// 0 <= dist < w0 (window), KIND 2 keeps dist >= w0 (the far pairs).  Masked
// scores become -inf.
template <int KIND>
__device__ inline void mask_tile(f32x16* s, int myrow, int j0, int w0, int g) {
  const int d0 = myrow - j0 - 8 * g;
#pragma unroll
  for (int sb = 0; sb < 2; ++sb)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      // dist = myrow - (j0 + key) = d0 - c with the lane-independent part c
      // of the key offset; the window test 0 <= dist < w0 is one unsigned
      // compare
      const int c = key_of(sb, i, 0);
      const bool keep = KIND == 0 ? d0 >= c : KIND == 2 ? d0 - w0 >= c : (uint32_t)(d0 - c) < (uint32_t)w0;
      s[sb][i] = keep ? s[sb][i] : -INFINITY;
    }
}

// Online softmax on raw scores s (masked entries -inf), first half: the row
// maximum and the lazy rescale of the accumulators when the stabiliser moves.
// Returns -m (the exp2 bias) for the second half.
__device__ inline float softmax_max(const f32x16* s, PassState& st, f32x16* o, float sl2) {
  float mx = -INFINITY;
#pragma unroll
  for (int sb = 0; sb < 2; ++sb)
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[sb][i]);
  mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * sl2;        // sl2 > 0
  const bool raise = mx > st.m + RESCALE_LOG2;          // false for an all-masked row
  if (__any(raise)) {
    const float mn = raise ? mx : st.m;
    const float a = st.m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(st.m - mn);
    st.l *= a;
#pragma unroll
    for (int db = 0; db < 4; ++db) o[db] *= a;
    st.m = mn;
  }
  return st.m == -INFINITY ? 0.f : -st.m;
}

// Second half: p = exp2(s sl2 - m) written back into s, row sum into st.l.
__device__ inline void softmax_exp(f32x16* s, PassState& st, float sl2, float nb) {
  float sum = 0.f;
#pragma unroll
  for (int sb = 0; sb < 2; ++sb)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[sb][i], sl2, nb));
      s[sb][i] = p;
      sum += p;
    }
  st.l += sum;
}

struct TileSrc {
  const char* k;       // K rows of (kv head, sequence), row-major 256 B rows
  const char* v;       // V^T tiles of (kv head, sequence), 16 KiB [128][64] blocks
  const __bf16* klo;   // residual K rows (PRECISE), row p of the sequence
};

struct WaveRows {
  int iw;      // first row of the wave
  int myrow;   // this lane's row
  int w0;
};

// Does this wave have any (causal / window) pair in the key tile at j0?
template <int KIND>
__device__ inline bool wave_has_work(int j0, const WaveRows& wr) {
  if (j0 > wr.iw + 31 - (KIND == 2 ? wr.w0 : 0)) return false;
  if (KIND == 1 && j0 + BK - 1 < wr.iw - wr.w0 + 1) return false;
  return true;
}

template <int KIND>
__device__ inline bool wave_needs_mask(int j0, const WaveRows& wr) {
  if (KIND == 2) return j0 + BK - 1 > wr.iw - wr.w0;         // some pair has dist < w0
  bool m = j0 + BK - 1 > wr.iw;                              // some pair has dist < 0
  if (KIND == 1) m = m || (j0 < wr.iw + 31 - wr.w0 + 1);     // some pair has dist >= w0
  return m;
}

// A full flash pass over key tiles [t0, t1), software-pipelined within each
// wave: the MFMAs of S(t+1) = K_{t+1} Q^T are issued before the softmax of
// tile t, so that vector-ALU work overlaps them.  K and V^T tiles have two
// LDS buffers each; K runs two tiles ahead, V one.  Iteration t:
//   wait for K(t+1), V(t); barrier (every wave is done with S(t)'s K buffer
//   and PV(t-1)'s V buffer); DMA K(t+2) and V(t+1) into those buffers;
//   S(t+1); softmax(t); PV(t).
template <int KIND, bool PRECISE>
__device__ inline void run_pass(char* smem, const TileSrc& src, int t0, int t1, const bf16x8* qf,
                                const bf16x8* ql, PassState& st, f32x16* o, const WaveRows& wr,
                                float sl2, int wave, int lane) {
  const int g = lane >> 5;
  __syncthreads();                      // every wave is done with all buffers
  if (t0 >= t1) return;
  const DmaPlan plan = make_dma_plan(wave, lane);
  char* const kb0 = smem;
  char* const kb1 = smem + KT_BYTES;
  char* const vb0 = smem + 2 * KT_BYTES;
  char* const vb1 = smem + 2 * KT_BYTES + VT_BYTES;
  auto kbuf = [&](int t) { return ((t - t0) & 1) ? kb1 : kb0; };
  auto vbuf = [&](int t) { return ((t - t0) & 1) ? vb1 : vb0; };
  auto issue_kt = [&](int t) { issue_k(kbuf(t), src.k + (int64_t)t * BK * 256, plan, wave); };
  auto issue_vt = [&](int t) { issue_v(vbuf(t), src.v + (int64_t)t * (D * BK * 2), plan, wave); };
  auto scores = [&](int t, f32x16* s) {
    score_tile<PRECISE>(kbuf(t), qf, ql, PRECISE ? src.klo + (int64_t)t * BK * D : nullptr, lane, s);
  };
  auto finish = [&](int t, f32x16* s) {
    const int j0 = t * BK;
    if (wave_needs_mask<KIND>(j0, wr)) mask_tile<KIND>(s, wr.myrow, j0, wr.w0, g);
    const float nb = softmax_max(s, st, o, sl2);
    softmax_exp(s, st, sl2, nb);
    pv_tile(vbuf(t), s, lane, o);
  };
  issue_kt(t0);
  if (t0 + 1 < t1) issue_kt(t0 + 1);
  issue_vt(t0);
  wait_all_tiles();
  __syncthreads();
  f32x16 sa[2], sb[2];
  bool wa = wave_has_work<KIND>(t0 * BK, wr), wb = false;
  if (wa) scores(t0, sa);
  // two iterations per trip so the two score sets never need a copy
  for (int t = t0; t < t1; t += 2) {
    // ---- iteration t: S(t) in sa ----
    wait_all_tiles();                   // K(t+1) and V(t) landed
    __syncthreads();
    if (t + 2 < t1) issue_kt(t + 2);
    if (t + 1 < t1) {
      issue_vt(t + 1);
      wb = wave_has_work<KIND>((t + 1) * BK, wr);
      if (wb) scores(t + 1, sb);
    }
    if (wa) finish(t, sa);
    if (t + 1 >= t1) break;
    // ---- iteration t+1: S(t+1) in sb ----
    wait_all_tiles();
    __syncthreads();
    if (t + 3 < t1) issue_kt(t + 3);
    if (t + 2 < t1) {
      issue_vt(t + 2);
      wa = wave_has_work<KIND>((t + 2) * BK, wr);
      if (wa) scores(t + 2, sa);
    }
    if (wb) finish(t + 1, sb);
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

// Work item of a block: head h, sequence b, q tile qt (rows qt*128 ..).
// FIRST: q tile 0 of every sequence (split-operand scores).  Otherwise q
// tiles >= 1 in the heavy-first, XCD-grouped order of JlSched.
template <bool FIRST>
__device__ inline bool block_item(const JlSched& sc, int Hq, int* h, int* b, int* qt) {
  const int n = blockIdx.x;
  if (FIRST) {
    *b = n / Hq;
    *h = sc.head_order[n % Hq];
    *qt = 0;
    return true;
  }
  int u;
  if (sc.xcd_heads > 0) {
    const int slot = n / sc.nxcd, s = n - slot * sc.nxcd;
    u = slot / sc.xcd_heads;
    *h = sc.head_order[s * sc.xcd_heads + slot % sc.xcd_heads];
  } else {
    u = n / Hq;
    *h = sc.head_order[n % Hq];
  }
  if (u >= sc.total_units) return false;
  unit_to_tile(sc, u, b, qt);
  return true;
}

struct PrefillArgs {
  const __bf16* q;    // the caller's [T][Hq][128] query, rotated by the kernels (rope_q)
  const __bf16* kb;
  const __bf16* kr;
  const __bf16* vt;
  const __bf16* kb_lo;
  const __bf16* kr_lo;
  __bf16* out;        // [T][Hq][128] bf16
  float* lse;         // [Hq][T] or nullptr
  float* o1;          // [Hq][nseq * JL_LO_ROWS][128] fp32: normalised pass 1 output of the first rows
  float* o2;          // [Hq][T][128] fp32: normalised pass 2 output (rows from JL_LO_ROWS on: see o2_slot)
  float* o3;          // [Hq][T][128] fp32: pass 3's accumulator (scaled by exp2(-m3)), rows from JL_LO_ROWS on (as o2)
  float* lse1;        // [Hq][nseq * JL_LO_ROWS]: pass 1 LogSumExp of the first rows (log2 units)
  float* lse2;        // [Hq][T]: pass 2 LogSumExp (log2 units)
  float2* ml3;        // [Hq][T]: pass 3's stabiliser m3 (log2 units) and sum, rows from JL_LO_ROWS on
  int64_t total;
  int64_t t_pad;
  int64_t w0;
  int Hq;
  int disjoint;       // far-only pass + window pass instead of the three passes (rows >= 128)
  float sl2;          // factor from score products to log2 units (1: q is pre-scaled)
  float qscale;       // softmax scale * log2(e), applied to q before its rotation and rounding
  JlFreqs fr;         // RoPE turn fractions theta_m / (2 pi), 0.64 fixed point
};

// The lane's 64 channels of one query row in the MFMA B-operand layout
// (qf[kb] holds channels kb * 16 + 8 g .. + 7, g = lane / 32), scaled by qscale,
// rotated by RoPE at position pos and rounded to bf16 (technical summary on
// gist.science, Methodology item 1: q and k rotated at their base or their
// aliased positions), with the scaling, pair rotation and rounding of the
// RoPE pre-pass for k.  Channel m < 64 of qf[kb] (kb < 4) and its pair
// partner m + 64 in qf[kb + 4] sit in the same lane.  Rows past the sequence
// end (valid false) are zero.  With LO (the split operands of a sequence's
// first rows) ql receives the rounding residuals bf16(y - bf16(y)) and the
// angles come from the pre-pass's exact sin/cos, so both are bitwise what a
// pre-pass over q would write; otherwise from the hardware sine and cosine,
// within 1.3e-7 of the exact values (far below q's bf16 rounding).
// The rotation of the caller's bf16 channels x (x[kb]: channels kb * 16 + 8 g
// .. + 7 of the row, as load_q_raw reads them).
template <bool LO>
__device__ inline void rotate_q(bf16x8* qf, bf16x8* ql, const bf16x8* x, bool valid, int pos,
                                const PrefillArgs& A, int g) {
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float s, c;
      const uint64_t tf = A.fr.turn_frac[kb * 16 + g * 8 + e];
      if constexpr (LO) {
        jl_rope_sincos(pos, tf, &s, &c);
      } else {
        // the hardware sine and cosine take the angle in turns, which the
        // fixed-point angle already is (top 32 bits: a turn fraction in
        // [-1/2, 1/2))
        const float t = (float)(int32_t)(jl_angle_turns(pos, tf) >> 32) * (1.0f / 4294967296.0f);
        s = __builtin_amdgcn_sinf(t);
        c = __builtin_amdgcn_cosf(t);
      }
      const float x1 = valid ? (float)x[kb][e] * A.qscale : 0.f;
      const float x2 = valid ? (float)x[kb + 4][e] * A.qscale : 0.f;
      float y1, y2;
      jl_rot_pair(x1, x2, c, s, &y1, &y2);
      const __bf16 h1 = (__bf16)y1, h2 = (__bf16)y2;
      qf[kb][e] = h1;
      qf[kb + 4][e] = h2;
      if constexpr (LO) {
        ql[kb][e] = (__bf16)(y1 - (float)h1);
        ql[kb + 4][e] = (__bf16)(y2 - (float)h2);
      }
    }
}

__device__ inline void load_q_raw(bf16x8* x, const __bf16* rowp, int g) {
#pragma unroll
  for (int kb = 0; kb < 8; ++kb) x[kb] = *(const bf16x8*)(rowp + kb * 16 + g * 8);
}

template <bool LO>
__device__ inline void rope_q(bf16x8* qf, bf16x8* ql, const __bf16* rowp, bool valid, int pos,
                              const PrefillArgs& A, int g) {
  bf16x8 x[8];
  load_q_raw(x, rowp, g);
  rotate_q<LO>(qf, ql, x, valid, pos, A, g);
}

struct BlockCtx {
  int h, b, kvh, L, i0, w0, wave, lane, g;
  int64_t s0;
  bool only1, only2;
  int tiles_end, tw0;
  WaveRows wr;
  TileSrc base_src, rem_src;
  int64_t lrows, lo_base;
};

__device__ inline bool make_ctx(const PrefillArgs& A, const JlHeadMap& hm, const JlSeqs& seqs,
                                int h, int b, int qt, BlockCtx* c) {
  c->h = h;
  c->b = b;
  c->L = seqs.len[b];
  c->i0 = qt * BQ;
  if (c->i0 >= c->L) return false;
  const int tid = threadIdx.x;
  // wave index in a scalar register: the LDS destination of global_load_lds
  // (M0) must be wave-uniform
  c->wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  c->lane = tid & 63;
  c->g = c->lane >> 5;
  c->kvh = hm.kv_of[h];
  c->s0 = seqs.start[b];
  c->w0 = A.w0 > (int64_t)c->L ? c->L : (int)A.w0;
  c->only1 = c->w0 >= c->L;                       // every pair local: pass 1 alone
  c->only2 = seqs.G[b] == 1 && !c->only1;          // remote grid == base grid: pass 2 alone
  const int iw = c->i0 + c->wave * 32;
  c->wr = WaveRows{iw, iw + (c->lane & 31), c->w0};
  c->tiles_end = min((c->i0 + BQ + BK - 1) / BK, (c->L + BK - 1) / BK);
  c->tw0 = (c->i0 - c->w0 + 1) > 0 ? (c->i0 - c->w0 + 1) / BK : 0;   // first window tile
  c->lrows = (int64_t)seqs.nseq * JL_LO_ROWS;
  c->lo_base = (int64_t)b * JL_LO_ROWS;
  const int64_t vtiles = seqs.vt_cols / 64;
  const char* vbase = (const char*)(A.vt + ((int64_t)c->kvh * vtiles + seqs.vstart[b] / 64) * (D * 64));
  c->base_src = TileSrc{(const char*)(A.kb + ((int64_t)c->kvh * A.t_pad + c->s0) * D), vbase,
                        A.kb_lo + ((int64_t)c->kvh * c->lrows + c->lo_base) * D};
  c->rem_src = TileSrc{(const char*)(A.kr + ((int64_t)c->kvh * A.t_pad + c->s0) * D), vbase,
                       A.kr_lo + ((int64_t)c->kvh * c->lrows + c->lo_base) * D};
  return true;
}

// The block's query row of this lane, rotated at its base (REMOTE false) or
// aliased position; rows past the sequence end load row L - 1 and become zero.
template <bool PRECISE, bool REMOTE>
__device__ inline void load_q_pair(bf16x8* qf, bf16x8* ql, const PrefillArgs& A, const JlSeqs& seqs,
                                   const BlockCtx& c) {
  const bool valid = c.wr.myrow < c.L;
  const int row = valid ? c.wr.myrow : c.L - 1;
  const int pos = REMOTE ? jl_remote_pos(row, seqs.G[c.b]) : row;
  rope_q<PRECISE>(qf, ql, A.q + ((c.s0 + row) * A.Hq + c.h) * D, valid, pos, A, c.g);
}

// o (unnormalised, lane holds channels db*32 + 8*(i/4) + 4*g + i%4 of its row)
// * scale -> bf16 output row.
__device__ inline void store_out(const PrefillArgs& A, const BlockCtx& c, const f32x16* o, float scale) {
  __bf16* orow = A.out + ((c.s0 + c.wr.myrow) * A.Hq + c.h) * D;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      bf16x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = (__bf16)(o[db][4 * q4 + e] * scale);
      *(bf16x4*)(orow + db * 32 + 8 * q4 + 4 * c.g) = w;
    }
}

// ---- one flash pass per launch --------------------------------------------
// ROLE 0: pass 2 (remote q/k, causal, all key tiles).  For G = 1 sequences it
//         is the whole result; otherwise it leaves (o2, lse_2) in workspace.
// ROLE 1: pass 1 (base q/k, window tiles).  For w0 >= L it is the whole
//         result; otherwise it leaves (o1, lse_1) in workspace.
// ROLE 2: pass 3 (remote q/k, window tiles), then the inclusion-exclusion
//         merge of the three (o_k, lse_k) into the output.
// o_k are stored normalised in fp32 and lse_k in log2 units.
template <int ROLE, bool FIRST>
__global__ void __launch_bounds__(NT, 2) prefill_pass_kernel(PrefillArgs A, JlHeadMap hm, JlSeqs seqs,
                                                             JlSched sc) {
  constexpr int KIND = ROLE == 0 ? 0 : 1;
  __shared__ __align__(1024) char smem[2 * KT_BYTES + 2 * VT_BYTES];
  int h, b, qt;
  if (!block_item<FIRST>(sc, A.Hq, &h, &b, &qt)) return;
  BlockCtx c;
  if (!make_ctx(A, hm, seqs, h, b, qt, &c)) return;
  if (ROLE == 0 && c.only1) return;
  if (ROLE == 1 && c.only2) return;
  if (ROLE == 2 && (c.only1 || c.only2)) return;
  bf16x8 qf[8];
  bf16x8 ql[FIRST ? 8 : 1];
  if (ROLE == 1) load_q_pair<FIRST, false>(qf, ql, A, seqs, c);
  else load_q_pair<FIRST, true>(qf, ql, A, seqs, c);
  f32x16 o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) o[db] = f32x16{};
  PassState st{-INFINITY, 0.f};
  const int t0 = ROLE == 0 || c.only1 ? 0 : c.tw0;
  run_pass<KIND, FIRST>(smem, ROLE == 1 ? c.base_src : c.rem_src, t0, c.tiles_end, qf, ql, st, o, c.wr,
                        A.sl2, c.wave, c.lane);
  const float l = st.l + __shfl_xor(st.l, 32, 64);
  if (c.wr.myrow >= c.L) return;
  const int64_t ridx = (int64_t)c.h * A.total + c.s0 + c.wr.myrow;
  // pass 1's output of the first rows: [Hq][nseq * JL_LO_ROWS] rows
  const int64_t lidx = (int64_t)c.h * c.lrows + c.lo_base + c.wr.myrow;
  if constexpr (ROLE != 2) {
    // lse_k in log2 units; an empty pass (w0 = 0 leaves pass 1 without keys)
    // has lse = -inf and weight 0 in the merge
    const float lam = l > 0.f ? st.m + __log2f(l) : -INFINITY;
    if ((ROLE == 0 && c.only2) || (ROLE == 1 && c.only1)) {
      store_out(A, c, o, 1.f / l);
      if (A.lse != nullptr && c.g == 0) A.lse[ridx] = lam * LN2;
      return;
    }
    float* orow = ROLE == 0 ? A.o2 + ridx * D : A.o1 + lidx * D;
    const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        *(float4*)(orow + db * 32 + 8 * q4 + 4 * c.g) =
            make_float4(o[db][4 * q4] * inv, o[db][4 * q4 + 1] * inv, o[db][4 * q4 + 2] * inv,
                        o[db][4 * q4 + 3] * inv);
    if (c.g == 0) {
      if (ROLE == 0) A.lse2[ridx] = lam;
      else A.lse1[lidx] = lam;
    }
  } else {
    // ---- merge: M = max(lse_1, lse_2), z_k = 2^(lse_k - M) ----
    const float lam1 = A.lse1[lidx];
    const float lam2 = A.lse2[ridx];
    const float lam3 = l > 0.f ? st.m + __log2f(l) : -INFINITY;
    const float M = fmaxf(lam1, lam2);
    const float z1 = __builtin_amdgcn_exp2f(lam1 - M);
    const float z2 = __builtin_amdgcn_exp2f(lam2 - M);
    const float z3 = __builtin_amdgcn_exp2f(lam3 - M);
    const float c3 = l > 0.f ? __builtin_amdgcn_exp2f(st.m - M) : 0.f;   // z3 o3 = c3 * A3
    // the remote-only mass z2 - z3 is exactly 0 for rows without remote pairs
    // (passes 2 and 3 then see identical scores) and never counted negative
    const float far = z2 - z3;
    const float Z = z1 + fmaxf(far, 0.f);
    const float inv = 1.f / Z;
    const float* o1row = A.o1 + lidx * D;
    const float* o2row = A.o2 + ridx * D;
    __bf16* orow = A.out + ((c.s0 + c.wr.myrow) * A.Hq + c.h) * D;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d0 = db * 32 + 8 * q4 + 4 * c.g;
        const float4 v1 = *(const float4*)(o1row + d0);
        const float4 v2 = *(const float4*)(o2row + d0);
        const float o1v[4] = {v1.x, v1.y, v1.z, v1.w};
        const float o2v[4] = {v2.x, v2.y, v2.z, v2.w};
        bf16x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float far_num = far > 0.f ? z2 * o2v[e] - c3 * o[db][4 * q4 + e] : 0.f;
          w[e] = (__bf16)((z1 * o1v[e] + far_num) * inv);
        }
        *(bf16x4*)(orow + d0) = w;
      }
    if (A.lse != nullptr && c.g == 0) A.lse[ridx] = (M + __log2f(Z)) * LN2;
  }
}

// ---- eight-wave ping-pong pass kernel (q rows >= 128) ---------------------
// One workgroup = 8 waves = 256 query rows [r0, r0 + 256) of one head, with
// r0 = 128 + 256 u (rows 0..127 of a sequence are the split-operand tile of
// the kernel above).  Waves 0-3 (group A) own rows r0 .. r0 + 127 and waves
// 4-7 (group B) rows r0 + 128 .. r0 + 255; wave w runs on SIMD w % 4, so each
// SIMD holds one wave of each group.  Work advances in half-steps separated
// by workgroup barriers; in every half-step one group issues matrix work
// (S(k) = K_k Q^T and O += V_{k-1} P_{k-1}^T, 32 MFMAs per wave) while the
// other runs the softmax of its last score tile on the vector ALU, and the
// roles swap at the next half-step.  The MFMA pipe of a SIMD therefore always
// has one wave feeding it while the other wave's exp / max / convert work
// runs beside it.
//
// Half-step h (h = 0 .. 2n+1 for n key tiles): group g is in phase
// ph = h - g; an even phase 2k is the matrix phase of tile k (S(k), PV(k-1)),
// an odd phase 2k+1 the softmax of tile k.  K_k is read in half-steps 2k and
// 2k+1 and V_k in 2k+2 and 2k+3.  Group B copies K_k into LDS at the start of
// half-step 2k - 2 and group A copies V_k at the start of half-step 2k + 1,
// each during its own softmax phase; each waits for its copies at the end of
// an odd half-step, before the barrier ahead of the tile's first reader, so
// two buffers of each suffice.
constexpr int PP_NT = 512;
constexpr int PP_BQ = 256;
// a tile's 16-byte pieces are spread over the four waves of the group that
// copies it (group B the K tiles, group A the V^T tiles)
constexpr int PP_K_PER_WAVE = (KT_PIECES + 3) / 4;   // 5
constexpr int PP_V_PER_WAVE = (VT_PIECES + 3) / 4;   // 5
constexpr int BUF_RSRC_WORD3 = 0x00020000;           // raw buffer, 32-bit data format

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct PpDma {
  uint32_t koff[PP_K_PER_WAVE];
  uint32_t voff[PP_V_PER_WAVE];
};

__device__ inline PpDma make_pp_dma(int wave, int lane) {
  PpDma p;
#pragma unroll
  for (int i = 0; i < PP_K_PER_WAVE; ++i) {
    const int n = min((wave & 3) + 4 * i, KT_PIECES - 1);
    const int off = n * 1024 + lane * 16;
    const int r = off / KP, cb = off - r * KP;
    p.koff[i] = (uint32_t)(r * 256 + (cb < 256 ? cb : 0));
  }
#pragma unroll
  for (int i = 0; i < PP_V_PER_WAVE; ++i) {
    const int n = min((wave & 3) + 4 * i, VT_PIECES - 1);
    const int off = n * 1024 + lane * 16;
    const int r = off / VP, cb = off - r * VP;
    p.voff[i] = (uint32_t)(r * 128 + (cb < 128 ? cb : 0));
  }
  return p;
}

typedef __attribute__((address_space(3))) char lds_char;

__device__ inline int64_t uniform_i64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)(uint64_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Copies one 16 KiB source tile (byte offset toff from the resource base)
// into an LDS tile buffer: the per-lane offsets are fixed, the tile offset is
// a scalar, so no vector address arithmetic is spent per tile.
template <int PER_WAVE, int PIECES>
__device__ inline void pp_issue(lds_char* buf, __amdgpu_buffer_rsrc_t rs, const uint32_t* off, uint32_t toff,
                                int wave) {
#pragma unroll
  for (int i = 0; i < PER_WAVE; ++i) {
    const int n = min(wave + 4 * i, PIECES - 1);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(buf + n * 1024), 16, off[i], (int)toff, 0, 0);
  }
}

// Phase boundary: no instruction may be scheduled across it (the matrix and
// softmax phases of the two groups must stay where the barriers put them).
__device__ inline void pp_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}
__device__ inline void pp_wait_copies() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

__device__ inline float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Output channels of a row in 16-byte pieces.  Lanes t and t + 32 (g = 0, 1)
// hold the same row; for a slot pair (q4 = 2m, 2m + 1) lane g has channels
// base + 4g .. + 3 of slot 2m in a and base + 8 + 4g .. + 3 of slot 2m + 1 in
// b.  One swap of the upper half of a with the lower half of b gives lane g
// the 8 channels base + 8g .. + 7, so that one 16-byte store per lane covers
// 32 contiguous bytes of the row where two 8-byte stores covered 16.
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
__device__ inline u32x4 pair_channels(u32x2 a, u32x2 b) {
  const auto lo = __builtin_amdgcn_permlane32_swap(a[0], b[0], false, false);
  const auto hi = __builtin_amdgcn_permlane32_swap(a[1], b[1], false, false);
  return u32x4{lo[0], hi[0], lo[1], hi[1]};
}

__device__ inline float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Row state of a flash pass in the ping-pong kernel.  Scores arrive in log2
// units (q is pre-scaled) and already shifted by -m: the first MFMA of each
// score chain takes the register tile cb = (-m, ..., -m) as its accumulator
// input, so the softmax exponentiates the MFMA output directly.  cb lives
// across tiles and is rewritten only when the stabiliser moves, which keeps
// both the shift and its set-up out of the per-tile vector-ALU work (the
// vector ALU and the MFMA pipe of one SIMD hardly overlap).
struct PpState {
  float m;      // stabiliser (log2 units), identical in lanes l and l ^ 32; -inf before any key
  float l;      // this lane's partial sum of the bf16 probabilities
  f32x16 cb;    // (-m, ..., -m), 0 while the row has no stabiliser: the score MFMAs' accumulator input
};

// -m, or 0 while the row has no stabiliser
__device__ inline float pp_shift(const PpState& st) { return st.m == -INFINITY ? 0.f : -st.m; }

// S^T of one 64-key tile (same layout as score_tile): s[sb] holds keys
// sb*32 + 16*(i/8) + 8*g + (i%8) of this lane's query row.
__device__ inline void pp_scores(const lds_char* kt, const bf16x8* qf, const f32x16& cb, int lane, f32x16* s) {
  const int g = lane >> 5;
  const lds_char* base = kt + swap23(lane & 31) * KP + g * 16;
  f32x16 a0 = cb, a1 = cb;
#pragma unroll
  for (int kb = 0; kb < 8; ++kb) {
    const bf16x8 k0 = *(const __attribute__((address_space(3))) bf16x8*)(base + kb * 32);
    const bf16x8 k1 = *(const __attribute__((address_space(3))) bf16x8*)(base + 32 * KP + kb * 32);
    a0 = mfma(k0, qf[kb], a0);
    a1 = mfma(k1, qf[kb], a1);
  }
  s[0] = a0;
  s[1] = a1;
}

// o[db] += V^T[db*32 .. +31][keys] * P^T, P already bf16
__device__ inline void pp_pv(const lds_char* vt, const bf16x8* p, int lane, f32x16* o) {
  const lds_char* base = vt + (lane & 31) * VP + (lane >> 5) * 16;
#pragma unroll
  for (int sb = 0; sb < 2; ++sb)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int c = sb * 4 + hh * 2;
#pragma unroll
      for (int db = 0; db < 4; ++db)
        o[db] = mfma(*(const __attribute__((address_space(3))) bf16x8*)(base + db * 32 * VP + c * 16),
                     p[2 * sb + hh], o[db]);
    }
}

// p = bf16(exp2(s + shift)) for the 32 scores of a lane (SHIFT false: shift
// is 0 and not applied); returns the sum of the fp32 values, accumulated in
// four independent chains of plain adds.  The sum is not taken with
// v_dot2c_f32_bf16 over the packed bf16 values: on gfx950 that instruction
// waits for the matrix pipe, and issued beside another wave's MFMAs it ran
// about seven times slower than an add in a micro-benchmark (38 cycles per
// dot2 against 5.6 alone).  In this kernel the two forms timed the same; the
// adds sum the fp32 weights exactly as they are, before their bf16 rounding.
template <bool SHIFT>
__device__ inline float pp_exp_tile(const f32x16* s, float shift, bf16x8* p) {
  float sum[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int sb = 0; sb < 2; ++sb)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      bf16x8 v;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float e = __builtin_amdgcn_exp2f(SHIFT ? s[sb][8 * hh + j] + shift : s[sb][8 * hh + j]);
        v[j] = (__bf16)e;
        sum[j & 3] += e;
      }
      p[2 * sb + hh] = v;
    }
  return (sum[0] + sum[1]) + (sum[2] + sum[3]);
}

// Largest probability a tile may produce before the stabiliser is moved.
// Any m keeps the result exact (lse = m + log2 l); the bound only keeps p,
// l and the accumulators far from fp32 overflow.
constexpr float PP_SUM_LIMIT = 4294967296.f;   // 2^32

// Softmax of one tile without a row maximum in the common case: the scores
// come shifted by the current stabiliser, so p = exp2(s) directly (done by
// the caller, tsum = this lane's tile sum).  The wave takes the exact path instead when a lane's tile
// sum exceeds 2^32 (a score more than ~27 above m) or a row has no stabiliser
// yet: row maximum, rescale of the accumulators, new stabiliser,
// exponentials again.
__device__ inline void pp_settle(const f32x16* s, bf16x8* p, PpState& st, f32x16* o, float tsum) {
  if (__builtin_expect(__all(tsum <= PP_SUM_LIMIT && st.m != -INFINITY), 1)) {
    st.l += tsum;
    return;
  }
  const float bias = pp_shift(st);                       // what the score MFMAs added
  float mx = -INFINITY;
#pragma unroll
  for (int sb = 0; sb < 2; ++sb)
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[sb][i]);
  mx = pair_max(mx);
  if (mx != -INFINITY) {
    const float mn = fmaxf(st.m, mx - bias);             // exact row maximum so far
    if (mn > st.m) {
      const float a = st.m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(st.m - mn);
      st.l *= a;
#pragma unroll
      for (int db = 0; db < 4; ++db) o[db] *= a;
      st.m = mn;
    }
  }
  const float nb = pp_shift(st);
#pragma unroll
  for (int i = 0; i < 16; ++i) st.cb[i] = nb;
  st.l += pp_exp_tile<true>(s, nb - bias, p);
}

__device__ inline void pp_softmax(const f32x16* s, bf16x8* p, PpState& st, f32x16* o) {
  pp_settle(s, p, st, o, pp_exp_tile<false>(s, 0.f, p));
}

// Instruction order of a matrix phase with NM MFMAs, each fed by one LDS
// read: the first DEPTH reads go out ahead, then every MFMA is followed by
// the read DEPTH positions later, so LDS latency hides behind the MFMAs.
template <int NM, int DEPTH>
__device__ inline void pp_mfma_order() {
  __builtin_amdgcn_sched_group_barrier(0x100, DEPTH, 0);   // LDS reads
#pragma unroll
  for (int i = 0; i < NM - DEPTH; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);     // MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);     // LDS read
  }
  __builtin_amdgcn_sched_group_barrier(0x008, DEPTH, 0);
}

constexpr int PP_READ_DEPTH = 8;

struct PpTiles {
  lds_char* lds;
  __amdgpu_buffer_rsrc_t rk, rv;
  PpDma plan;
  int t0, n, wave;
};


__device__ inline lds_char* pp_kbuf(const PpTiles& T, int k) { return T.lds + (k & 1) * KT_BYTES; }
__device__ inline lds_char* pp_vbuf(const PpTiles& T, int k) {
  return T.lds + 2 * KT_BYTES + (k & 1) * VT_BYTES;
}

// copies issued by group B at half-step 2j: K_{j+1} (if any).  The K and
// V^T copies of a tile are split between the groups (B copies K, A copies
// V^T): a wave that issues copies is held at each issue while the vector
// memory unit works through the queue, and with all ten pieces of a tile in
// one group's softmax phase that phase outlasted the other group's matrix
// phase (same-box A/B: the split is 2.4% faster on the whole prefill).
__device__ inline void pp_copies(const PpTiles& T, int j) {
  if (j + 1 < T.n)
    pp_issue<PP_K_PER_WAVE, KT_PIECES>(pp_kbuf(T, j + 1), T.rk, T.plan.koff,
                                       (uint32_t)(T.t0 + j + 1) * (BK * 256), T.wave & 3);
}
// copies issued by group A at half-step 2j+1: V_j, at the start of its
// softmax phase, waited for at the end of that phase (issued at the end
// instead, the copy's latency is exposed: 9% slower on the whole prefill; one
// tile ahead into a third V^T buffer was 1.3% slower than this, same box)
__device__ inline void pp_copies_v(const PpTiles& T, int j) {
  pp_issue<PP_V_PER_WAVE, VT_PIECES>(pp_vbuf(T, j), T.rv, T.plan.voff, (uint32_t)(T.t0 + j) * (D * BK * 2),
                                     T.wave & 3);
}

template <int KIND>
__device__ inline void pp_softmax_tile(const PpTiles& T, int k, f32x16* s, bf16x8* p, PpState& st, f32x16* o,
                                       const WaveRows& wr, int g) {
  const int j0 = (T.t0 + k) * BK;
  if (!wave_has_work<KIND>(j0, wr)) {
    // no pair of the wave's rows in this tile: P = 0, the row state is unchanged
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = bf16x8{};
    return;
  }
  if (wave_needs_mask<KIND>(j0, wr)) mask_tile<KIND>(s, wr.myrow, j0, wr.w0, g);
  pp_softmax(s, p, st, o);
}

// Matrix phase of a wave: S_k (shifted by the current stabiliser) and O += V_{k-1}
// P_{k-1}^T.  It runs at raised wave priority: an MFMA then issues as soon as
// the pipe takes it, once per 8 passes, and the softmax-phase wave beside it
// on the SIMD fills every other issue slot.  With the priority on the softmax
// side instead (or on neither), vector-ALU bursts hold back MFMA issue and the
// pipe idles (measured: about 2% of the whole prefill).
__device__ inline void pp_matrix(const PpTiles& T, int k, bool pv, const bf16x8* qf, const PpState& st, f32x16* s,
                                 const bf16x8* p, f32x16* o, int lane) {
  __builtin_amdgcn_s_setprio(2);
  pp_scores(pp_kbuf(T, k), qf, st.cb, lane, s);
  if (pv) {
    pp_pv(pp_vbuf(T, k - 1), p, lane, o);
    pp_mfma_order<32, PP_READ_DEPTH>();
  } else {
    pp_mfma_order<16, PP_READ_DEPTH>();
  }
  __builtin_amdgcn_s_setprio(0);
}

// The two groups run mirrored straight-line loops with the same number of
// barriers (half-step h: group A is in its matrix phase for even h, group B
// for odd h).  K_k is read in half-steps 2k, 2k+1 and V_k in 2k+2, 2k+3.
// Group B copies K_{k+1} at the start of half-step 2k (ahead of its softmax
// phase), into the buffer whose last readers finished at half-step 2k-1, and
// waits for it at the end of half-step 2k+1 (after its matrix phase), in time
// for group A's matrix phase at 2k+2.  Group A copies V_k at the start of
// half-step 2k+1 (its softmax phase of tile k) into the buffer of V_{k-2},
// whose last reader finished at half-step 2k-1, and waits for it at the end
// of that half-step, in time for its matrix phase at 2k+2.  Tiles in
// which a wave has no pair (the last two causal tiles of group A, the first
// two window tiles of group B) keep their MFMAs, which keeps the loops free
// of per-wave branches around register-resident state; their softmax only
// writes P = 0.  Both loops produce and consume S within one iteration and
// carry only P across the back edge: with S carried instead (group B's
// natural order), the register allocator copied the stabiliser tile and one
// score half every tile, 16 extra vector moves (measured: 2% of the prefill).
// Group B's loop is rotated for that: matrix phase, then the copies and
// softmax of the same tile.
// Group A's side of a pass (waves 0-3), from the copy of K_0 on.
template <int KIND>
__device__ inline void pp_walk_a(const PpTiles& T, const bf16x8* qf, PpState& st, f32x16* o, const WaveRows& wr,
                                 int lane) {
  const int n = T.n;
  const int g = lane >> 5;
  f32x16 s[2];
  bf16x8 p[4];
  pp_issue<PP_K_PER_WAVE, KT_PIECES>(pp_kbuf(T, 0), T.rk, T.plan.koff, (uint32_t)T.t0 * (BK * 256), T.wave);
  pp_wait_copies();
  pp_barrier();
  pp_matrix(T, 0, false, qf, st, s, p, o, lane);
  pp_barrier();
  pp_copies_v(T, 0);
  pp_softmax_tile<KIND>(T, 0, s, p, st, o, wr, g);
  pp_wait_copies();
  pp_barrier();
  for (int j = 1; j < n; ++j) {
    pp_matrix(T, j, true, qf, st, s, p, o, lane);
    pp_barrier();
    pp_copies_v(T, j);
    pp_softmax_tile<KIND>(T, j, s, p, st, o, wr, g);
    pp_wait_copies();
    pp_barrier();
  }
  pp_pv(pp_vbuf(T, n - 1), p, lane, o);
  pp_mfma_order<16, PP_READ_DEPTH>();
  pp_barrier();
  pp_barrier();
}

// Group B's side of a pass (waves 4-7), with the same number of barriers.
template <int KIND>
__device__ inline void pp_walk_b(const PpTiles& T, const bf16x8* qf, PpState& st, f32x16* o, const WaveRows& wr,
                                 int lane) {
  const int n = T.n;
  const int g = lane >> 5;
  f32x16 s[2];
  bf16x8 p[4];
  pp_wait_copies();
  pp_barrier();
  pp_copies(T, 0);
  pp_barrier();
  pp_matrix(T, 0, false, qf, st, s, p, o, lane);
  pp_wait_copies();
  pp_barrier();
  if (n > 1) pp_copies(T, 1);
  pp_softmax_tile<KIND>(T, 0, s, p, st, o, wr, g);
  pp_barrier();
  for (int j = 1; j < n; ++j) {
    pp_matrix(T, j, true, qf, st, s, p, o, lane);
    pp_wait_copies();
    pp_barrier();
    if (j + 1 < n) pp_copies(T, j + 1);
    pp_softmax_tile<KIND>(T, j, s, p, st, o, wr, g);
    pp_barrier();
  }
  pp_pv(pp_vbuf(T, n - 1), p, lane, o);
  pp_mfma_order<16, PP_READ_DEPTH>();
  pp_barrier();
}

// One group's side of a pass: group A (waves 0-3) or group B.
template <int KIND, bool GA>
__device__ inline void pp_walk(const PpTiles& T, const bf16x8* qf, PpState& st, f32x16* o, const WaveRows& wr,
                               int lane) {
  if constexpr (GA) pp_walk_a<KIND>(T, qf, st, o, wr, lane);
  else pp_walk_b<KIND>(T, qf, st, o, wr, lane);
}

template <int KIND>
__device__ inline void pp_run(const PpTiles& T, const bf16x8* qf, PpState& st, f32x16* o, const WaveRows& wr,
                              int lane) {
  if (T.wave < 4) pp_walk_a<KIND>(T, qf, st, o, wr, lane);
  else pp_walk_b<KIND>(T, qf, st, o, wr, lane);
}

// Pass 1's normalised output of a 256-row tile, kept in LDS by ROLE 0 until
// its merge: 64 bf16 per lane, chunk c (8 values: channels 32 (c / 2) +
// 8 (c % 2) .. of the lane's slots) of thread t at (c * PP_NT + t) * 16
// bytes.  o1 enters the merge with a positive weight only (the cancelling
// pair is passes 2 and 3, kept in fp32), so bf16 holds it within the
// output's own rounding.  Before pass 1 ends, the same bytes of each thread
// hold its raw query row for the second rotation.
constexpr int O1_BYTES = PP_NT * 128;
// pass 1's log2-LSE of each thread's row, beside o1 (in LDS rather than in a
// register across the two later walks)
constexpr int LAM1_BYTES = PP_NT * 4;

// Pass 2's (or the far pass's) fp32 output of rows >= JL_LO_ROWS, as the
// 256-row kernel writes and reads it.  slab is the wave's first row.  A lane
// holds channels db*32 + 8*q4 + 4*g + 0..3 of its row in slot i = 4*db + q4.
// When all 32 rows of the wave lie in the sequence, the slab's 16 KB are in
// lane order instead of row order, slot i of lane t at (64 i + t) * 4 floats,
// so that each store and load instruction covers 1 KB of contiguous memory
// (row order puts 32 B of each of 32 rows in an instruction).  The last,
// partial 32 rows of a sequence stay row-ordered: a lane-ordered slab would
// run into the next rows.
__device__ inline float* o2_slot(float* slab, int lane, int i, bool lane_order) {
  return lane_order ? slab + (64 * i + lane) * 4
                    : slab + (lane & 31) * D + (i >> 2) * 32 + 8 * (i & 3) + 4 * (lane >> 5);
}

// The lane's 16 slots, all loads issued before any use: the merge stores bf16
// rows in between, and with the loads next to their uses the compiler kept
// each behind the previous store (it cannot prove the two arrays apart), one
// memory round trip per 16 bytes.
__device__ inline void pp_load_row(float4* v, const float* slab, int lane, bool lane_order) {
#pragma unroll
  for (int i = 0; i < 16; ++i) v[i] = *(const float4*)o2_slot((float*)slab, lane, i, lane_order);
}

// ROLE 0's walks for one wave group (GA: waves 0-3): pass 1 on the base
// grid (the whole attention when single), its output to LDS, then pass 3 on
// the remote grid, whose state is stored, then the far tiles, after which the
// state is pass 2's.  Each group runs its walks in its own branch: joining
// the groups between walks that carry the state made the register allocator
// spill it.
template <bool GA>
__device__ inline __attribute__((always_inline)) void pp_three_walks(
    const PrefillArgs& A, const PpTiles& T, bf16x8* qf, PpState& st, f32x16* o, const WaveRows& wr, int lane,
    bool single, bool live, bool q_valid, int q_row, int G, int64_t krow,
    __attribute__((address_space(3))) bf16x8* o1s, float* lam1s, int64_t slab_off, int L, int h, int64_t s0,
    int far_tiles) {
  const int g = lane >> 5;
  const int iw = wr.iw;
  pp_walk<1, GA>(T, qf, st, o, wr, lane);
  if (single) return;
  // pass 1 done: its log2-LSE and o1 (normalised, bf16) to LDS, o1 after the
  // raw query rows come back from there
  const float l1 = pair_sum(st.l);
  *lam1s = l1 > 0.f ? st.m + __log2f(l1) : -INFINITY;
  bf16x8 x[8];
  if (live) {
#pragma unroll
    for (int c = 0; c < 8; ++c) x[c] = o1s[c * PP_NT];
  }
  {
    const float inv = l1 > 0.f ? 1.f / l1 : 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      bf16x8 w;
#pragma unroll
      for (int e = 0; e < 8; ++e) w[e] = (__bf16)(o[c >> 1][8 * (c & 1) + e] * inv);
      o1s[c * PP_NT] = w;
    }
  }
  if (live) rotate_q<false>(qf, nullptr, x, q_valid, jl_remote_pos(q_row, G), A, g);
#pragma unroll
  for (int db = 0; db < 4; ++db) o[db] = f32x16{};
  st = PpState{-INFINITY, 0.f, f32x16{}};
  PpTiles T3 = T;
  T3.rk = __builtin_amdgcn_make_buffer_rsrc((void*)(A.kr + krow), 0, 0x7fffffff, BUF_RSRC_WORD3);
  pp_walk<1, GA>(T3, qf, st, o, wr, lane);
  if (live && wr.myrow < L) {
    // pass 3's state as it stands (a row without window pairs, w0 = 0,
    // stores m3 = -inf, l3 = 0 and a zero accumulator)
    const float l3 = pair_sum(st.l);
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        *(float4*)o2_slot(A.o3 + slab_off, lane, 4 * db + q4, iw + 32 <= L) =
            make_float4(o[db][4 * q4], o[db][4 * q4 + 1], o[db][4 * q4 + 2], o[db][4 * q4 + 3]);
    // both lanes of the row store the same (m3, l3), so that each reads
    // back its own store
    A.ml3[(int64_t)h * A.total + s0 + wr.myrow] = make_float2(st.m, l3);
  }
  T3.t0 = 0;
  T3.n = far_tiles;
  if (T3.n > 0) pp_walk<2, GA>(T3, qf, st, o, wr, lane);
}

// ROLE 0: all three passes of a 256-row tile and their merge.  Pass 1 (base
// q/k, window tiles) first, its normalised output kept in LDS.  Then passes
// 2 and 3 (remote q/k) from one walk over the key tiles: the walk takes the
// window tiles first under the window mask (0 <= i - j < w0), which is
// exactly pass 3, stores that running state (accumulator, stabiliser m3 and
// sum l3), and goes on over the far tiles under the far mask (i - j >= w0);
// the end state has seen every causal pair once, which is pass 2.  Pass 3
// thus shares pass 2's K/V tiles, scores and probabilities (only the few
// tiles that hold the window's lower edge are walked twice, once per mask).
// The inclusion-exclusion step then takes pass 3 from pass 2 in the frame of
// pass 2's stabiliser m2: with c = exp2(m3 - m2) (m only rises along the
// walk, so c <= 1), the far part is F = O2 - c O3 and l_far = l2 - c l3,
// which is z2 o2 - z3 o3 and z2 - z3 through the two passes' LogSumExp
// statistics (lam = m + log2 l), formed without the exp2 of large lam
// values.  The far mass is clamped at zero, and the merge with pass 1 is
// O = (z1 o1 + zf F) / (z1 + zf l_far), z1 = exp2(lam1 - M),
// zf = exp2(m2 - M), M = max(lam1, m2).  On a G = 1 sequence, or with
// w0 >= L, ROLE 0's first walk with the window set to L is the whole
// attention.
// The disjoint variant: ROLE 4 is the far pass alone (remote q/k, pairs with
// i - j >= w0 only, written to o2), and ROLE 5 is pass 1 merged with it,
// O = (z1 o1 + zf of) / (z1 + zf), two positive weights; sequences with
// w0 >= L run pass 1 over the whole causal range and write O directly; ROLE
// 0 then serves only the G = 1 sequences.
template <int ROLE>
__global__ void __launch_bounds__(PP_NT, 1) prefill_pp_kernel(PrefillArgs A, JlHeadMap hm, JlSeqs seqs,
                                                             JlSched sc) {
  static_assert(ROLE == 0 || ROLE == 4 || ROLE == 5, "pass roles of the 256-row kernel");
  constexpr int KIND = ROLE == 0 ? 0 : ROLE == 4 ? 2 : 1;
  constexpr bool BASE = ROLE == 0 || ROLE == 5;      // the first walk is pass 1, on the base grid
  __shared__ __align__(1024) char smem[2 * (KT_BYTES + VT_BYTES) + (ROLE == 0 ? O1_BYTES + LAM1_BYTES : 0)];
  int h, b, u;
  if (!block_item<false>(sc, A.Hq, &h, &b, &u)) return;
  // the work item is uniform over the block; say so, so that pointers built
  // from it (buffer resources in particular) live in scalar registers
  h = __builtin_amdgcn_readfirstlane(h);
  b = __builtin_amdgcn_readfirstlane(b);
  u = __builtin_amdgcn_readfirstlane(u);
  const int L = __builtin_amdgcn_readfirstlane(seqs.len[b]);
  const int r0 = JL_LO_ROWS + PP_BQ * (u - 1);
  if (r0 >= L) return;
  const bool only1 = A.w0 >= (int64_t)L;
  const bool only2 = seqs.G[b] == 1 && !only1;
  if (ROLE == 0 && A.disjoint && !only2) return;
  if (ROLE == 5 && only2) return;
  if (ROLE == 4 && (only1 || only2)) return;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int g = lane >> 5;
  const int kvh = __builtin_amdgcn_readfirstlane(hm.kv_of[h]);
  const int64_t s0 = uniform_i64(seqs.start[b]);
  // the window of the walk: w0, or L where it covers every causal pair (w0 >= L,
  // and ROLE 0's first walk on a G = 1 sequence, which is then the whole
  // attention: the two grids coincide)
  const int w0 = A.w0 > (int64_t)L || (ROLE == 0 && only2) ? L : (int)A.w0;
  const int iw = r0 + wave * 32;
  const WaveRows wr{iw, iw + (lane & 31), w0};
  const bool live = iw < L;             // waves past the end load nothing
  const int tiles_end = min((r0 + PP_BQ + BK - 1) / BK, (L + BK - 1) / BK);
  const int tw0 = (r0 - w0 + 1) > 0 ? (r0 - w0 + 1) / BK : 0;
  const int64_t vtiles = seqs.vt_cols / 64;
  const int64_t krow = ((int64_t)kvh * A.t_pad + s0) * D;
  const __bf16* ksrc = (BASE ? A.kb : A.kr) + krow;
  const __bf16* vsrc =
      A.vt + ((int64_t)kvh * vtiles + __builtin_amdgcn_readfirstlane(seqs.vstart[b]) / 64) * (D * 64);
  PpTiles T;
  lds_char* const lds = (lds_char*)smem;
  T.lds = lds;
  T.rk = __builtin_amdgcn_make_buffer_rsrc((void*)ksrc, 0, 0x7fffffff, BUF_RSRC_WORD3);
  T.rv = __builtin_amdgcn_make_buffer_rsrc((void*)vsrc, 0, 0x7fffffff, BUF_RSRC_WORD3);
  T.plan = make_pp_dma(wave, lane);
  T.wave = wave;
  bf16x8 qf[8];
  // this lane's query row (rows past the end: row L - 1's memory, zero
  // operands) and its positions on the two grids
  const bool q_valid = wr.myrow < L;
  const int q_row = q_valid ? wr.myrow : L - 1;
  const __bf16* q_src = A.q + ((s0 + q_row) * A.Hq + h) * D;
  // ROLE 0 rotates the same rows again for passes 3 and 2: the raw rows wait
  // in the LDS area of pass 1's output, which pass 1 does not touch, each
  // thread's 128 bytes where its own o1 chunks go (so no barrier is needed)
  __attribute__((address_space(3))) bf16x8* const o1s =
      (__attribute__((address_space(3))) bf16x8*)(lds + 2 * (KT_BYTES + VT_BYTES)) + tid;
  if (live) {
    bf16x8 x[8];
    load_q_raw(x, q_src, g);
    if constexpr (ROLE == 0) {
#pragma unroll
      for (int c = 0; c < 8; ++c) o1s[c * PP_NT] = x[c];
    }
    rotate_q<false>(qf, nullptr, x, q_valid,
                    BASE ? q_row : jl_remote_pos(q_row, __builtin_amdgcn_readfirstlane(seqs.G[b])), A, g);
  } else {
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) qf[kb] = bf16x8{};
  }
  f32x16 o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) o[db] = f32x16{};
  PpState st{-INFINITY, 0.f, f32x16{}};
  const int64_t slab_off = ((int64_t)h * A.total + s0 + iw) * D;
  // far pairs of the tile's rows end at key r0 + 255 - w0
  const int far_last = r0 + PP_BQ - 1 - w0;
  const int far_tiles = far_last < 0 ? 0 : min(tiles_end, far_last / BK + 1);
  float* const lam1s = (float*)(smem + 2 * (KT_BYTES + VT_BYTES) + O1_BYTES) + tid;   // ROLE 0
  if constexpr (ROLE == 0) {
    // pass 1, then passes 3 and 2 (the whole attention in one walk when
    // w0 >= L or G = 1)
    const bool single = only1 || only2;
    T.t0 = tw0;
    T.n = tiles_end - tw0;
    if (wave < 4)
      pp_three_walks<true>(A, T, qf, st, o, wr, lane, single, live, q_valid, q_row, seqs.G[b], krow, o1s, lam1s,
                           slab_off, L, h, s0, far_tiles);
    else
      pp_three_walks<false>(A, T, qf, st, o, wr, lane, single, live, q_valid, q_row, seqs.G[b], krow, o1s, lam1s,
                            slab_off, L, h, s0, far_tiles);
  } else {
    T.t0 = ROLE == 4 || only1 ? 0 : tw0;
    T.n = (ROLE == 4 ? far_tiles : tiles_end) - T.t0;
    if (T.n > 0) pp_run<KIND>(T, qf, st, o, wr, lane);
  }
  const float l = pair_sum(st.l);
  const float lam = l > 0.f ? st.m + __log2f(l) : -INFINITY;
  const int64_t ridx = (int64_t)h * A.total + s0 + wr.myrow;
  const bool row_ok = live && wr.myrow < L;
  float* const o2_slab = A.o2 + slab_off;
  const bool o2_lane_order = iw + 32 <= L;
  if (ROLE == 0 ? only1 || only2 : only1) {
    // the pass is the whole attention of the sequence
    if (!row_ok) return;
    __bf16* orow = A.out + ((s0 + wr.myrow) * A.Hq + h) * D;
    const float inv = 1.f / l;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int db = c >> 1;
      u32x2 w[2];
#pragma unroll
      for (int hq = 0; hq < 2; ++hq) {
        const int q4 = 2 * (c & 1) + hq;
        bf16x4 x;
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = (__bf16)(o[db][4 * q4 + e] * inv);
        w[hq] = __builtin_bit_cast(u32x2, x);
      }
      *(u32x4*)(orow + db * 32 + 16 * (c & 1) + 8 * g) = pair_channels(w[0], w[1]);
    }
    if (A.lse != nullptr && g == 0) A.lse[ridx] = lam * LN2;
    return;
  }
  if constexpr (ROLE == 0) {
    // the far part from passes 2 and 3 in pass 2's frame (c = exp2(m3 - m2)
    // <= 1: F = O2 - c O3, lf = l2 - c l3, the far mass clamped at zero),
    // merged with pass 1: M = max(lam1, m2), z1 = exp2(lam1 - M),
    // zf = exp2(m2 - M), O = (z1 o1 + zf F) / (z1 + zf lf)
    if (!row_ok) return;
    float4 s3[16];
    pp_load_row(s3, A.o3 + slab_off, lane, o2_lane_order);
    const float2 ml3 = A.ml3[ridx];
    const float c = ml3.x == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ml3.x - st.m);
    const float lf = l - c * ml3.y;
    const bool far = lf > 0.f;
    const float lam1 = *lam1s;
    const float M = fmaxf(lam1, st.m);                   // m2 is finite: pass 2 holds the diagonal
    const float z1 = __builtin_amdgcn_exp2f(lam1 - M);   // 0 when w0 = 0 (no window pair)
    const float zf = far ? __builtin_amdgcn_exp2f(st.m - M) : 0.f;
    const float Z = z1 + (far ? zf * lf : 0.f);
    const float inv = 1.f / Z;
    __bf16* orow = A.out + ((s0 + wr.myrow) * A.Hq + h) * D;
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) {
      const bf16x8 v1 = o1s[cc * PP_NT];
      const int db = cc >> 1;
      u32x2 w[2];
#pragma unroll
      for (int hq = 0; hq < 2; ++hq) {
        const int q4 = 2 * (cc & 1) + hq;
        const float4 v3 = s3[4 * db + q4];
        const float o3v[4] = {v3.x, v3.y, v3.z, v3.w};
        bf16x4 x;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          x[e] = (__bf16)((z1 * (float)v1[4 * hq + e] + zf * (o[db][4 * q4 + e] - c * o3v[e])) * inv);
        w[hq] = __builtin_bit_cast(u32x2, x);
      }
      *(u32x4*)(orow + db * 32 + 16 * (cc & 1) + 8 * g) = pair_channels(w[0], w[1]);
    }
    if (A.lse != nullptr && g == 0) A.lse[ridx] = (M + __log2f(Z)) * LN2;
  } else if constexpr (ROLE == 4) {
    // the far pass: rows without a far key (i < w0) store o = 0 and lam = -inf
    if (!row_ok) return;
    const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        *(float4*)o2_slot(o2_slab, lane, 4 * db + q4, o2_lane_order) =
            make_float4(o[db][4 * q4] * inv, o[db][4 * q4 + 1] * inv, o[db][4 * q4 + 2] * inv,
                        o[db][4 * q4 + 3] * inv);
    if (g == 0) A.lse2[ridx] = lam;
  } else if constexpr (ROLE == 5) {
    // pass 1 merged with the far part: window (base grid) and far (remote
    // grid) are two halves of one softmax, so both weights are positive
    if (!row_ok) return;
    const float lamf = A.lse2[ridx];
    const float M = fmaxf(lam, lamf);                    // lam is finite: the diagonal is in the window
    const float c1 = __builtin_amdgcn_exp2f(st.m - M);   // o carries exp2(s - st.m)
    const float zf = __builtin_amdgcn_exp2f(lamf - M);
    const float Z = __builtin_amdgcn_exp2f(lam - M) + zf;
    const float inv = 1.f / Z;
    __bf16* orow = A.out + ((s0 + wr.myrow) * A.Hq + h) * D;
    float4 vfs[16];
    pp_load_row(vfs, o2_slab, lane, o2_lane_order);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int db = c >> 1;
      u32x2 w[2];
#pragma unroll
      for (int hq = 0; hq < 2; ++hq) {
        const int q4 = 2 * (c & 1) + hq;
        const float4 vf = vfs[4 * db + q4];
        const float ofv[4] = {vf.x, vf.y, vf.z, vf.w};
        bf16x4 x;
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = (__bf16)((c1 * o[db][4 * q4 + e] + zf * ofv[e]) * inv);
        w[hq] = __builtin_bit_cast(u32x2, x);
      }
      *(u32x4*)(orow + db * 32 + 16 * (c & 1) + 8 * g) = pair_channels(w[0], w[1]);
    }
    if (A.lse != nullptr && g == 0) A.lse[ridx] = (M + __log2f(Z)) * LN2;
  }
}

}  // namespace

void jl_build_sched(const JlSeqs& seqs, const JlHeadMap& hm, int Hq, int nxcd, JlSched* sc) {
  // 256-row units of rows >= 128 of every sequence, grouped into levels of
  // equal count
  int c[JL_MAX_SEQS], perm[JL_MAX_SEQS], n = 0;
  for (int b = 0; b < seqs.nseq; ++b) {
    const int units = seqs.len[b] > JL_LO_ROWS ? (seqs.len[b] - JL_LO_ROWS + PP_BQ - 1) / PP_BQ : 0;
    if (units > 0) {
      c[n] = units;
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
  sc->nxcd = nxcd < 1 ? 1 : nxcd;
  sc->xcd_heads = (Hq % sc->nxcd == 0) ? Hq / sc->nxcd : 0;
}

hipError_t jl_launch_prefill_bf16(const JlPrefillWs& ws, const void* q, const JlFreqs& fr, float qscale,
                                  void* o, float* lse, int64_t total_tokens, int32_t Hq, int32_t Hkv,
                                  const JlHeadMap& hm, const JlSeqs& seqs, int64_t w0, float scale,
                                  int32_t max_len, bool disjoint, hipStream_t st) {
  (void)Hkv;
  (void)max_len;
  JlSched sc;
  jl_build_sched(seqs, hm, Hq, jl_device_shape().xcds, &sc);
  PrefillArgs A;
  A.q = (const __bf16*)q;
  A.kb = (const __bf16*)ws.kb;
  A.kr = (const __bf16*)ws.kr;
  A.vt = (const __bf16*)ws.vt;
  A.kb_lo = (const __bf16*)ws.kb_lo;
  A.kr_lo = (const __bf16*)ws.kr_lo;
  A.out = (__bf16*)o;
  A.lse = lse;
  A.o1 = (float*)ws.o1;
  A.o2 = (float*)ws.o2;
  A.o3 = (float*)ws.o3;
  A.lse1 = (float*)ws.lse1;
  A.lse2 = (float*)ws.lse2;
  A.ml3 = (float2*)ws.ml3;
  A.total = total_tokens;
  A.t_pad = ws.t_pad;
  A.w0 = w0;
  A.Hq = Hq;
  A.disjoint = disjoint ? 1 : 0;
  (void)scale;        // folded into q with log2 e (qscale) before its rotation
  A.sl2 = 1.f;
  A.qscale = qscale;
  A.fr = fr;
  bool any_p1 = false, any_p2 = false, any_p3 = false, any_only2 = false;
  for (int b = 0; b < seqs.nseq; ++b) {
    if (seqs.len[b] == 0) continue;
    const bool only1 = w0 >= (int64_t)seqs.len[b];
    const bool only2 = seqs.G[b] == 1 && !only1;
    any_p1 |= !only2;
    any_p2 |= !only1;
    any_p3 |= !only1 && !only2;
    any_only2 |= only2;
  }
  const unsigned nblk = (unsigned)sc.total_units * (unsigned)Hq;   // multiple of 8 when xcd_heads
  const unsigned nfirst = (unsigned)(seqs.nseq * Hq);
  // rows >= 128 in 256-row tiles: pass 1, then passes 2 and 3 from one walk,
  // and the merge, all in one workgroup; the first 128 rows of every
  // sequence in the split-operand kernel, pass by pass
  // disjoint: 256-row tiles run the far pass (ROLE 0 only for the G = 1
  // sequences), then pass 1 merged with it; the first 128 rows as above
  if (nblk && (!disjoint || any_only2)) prefill_pp_kernel<0><<<nblk, PP_NT, 0, st>>>(A, hm, seqs, sc);
  if (any_p2) prefill_pass_kernel<0, true><<<nfirst, NT, 0, st>>>(A, hm, seqs, sc);
  if (disjoint && any_p3 && nblk) prefill_pp_kernel<4><<<nblk, PP_NT, 0, st>>>(A, hm, seqs, sc);
  // profiling mark after the dominant launch of either form (all three passes
  // of rows >= 128, or the far pass)
  if (hipEvent_t mid = jl_profile_mid_event()) (void)hipEventRecord(mid, st);
  if (any_p1) {
    if (disjoint && nblk) prefill_pp_kernel<5><<<nblk, PP_NT, 0, st>>>(A, hm, seqs, sc);
    prefill_pass_kernel<1, true><<<nfirst, NT, 0, st>>>(A, hm, seqs, sc);
  }
  if (any_p3) prefill_pass_kernel<2, true><<<nfirst, NT, 0, st>>>(A, hm, seqs, sc);
  return hipGetLastError();
}
