// jl_internal.h - kernel parameter blocks and launcher declarations shared by
// the C ABI (jl_api.hip) and the kernels.  Not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/jetlong.h"
#include "jl_mapper.h"

#define JL_MAX_HEADS 128   // q heads per call
#define JL_MAX_HALF 64     // head_dim / 2

// Per-sequence schedule of one prefill call (packed varlen batch), built on
// the host from cu_seqlens and passed by value.
struct JlSeqs {
  int32_t nseq;
  int32_t any_remote;          // 1 if some sequence has G > 1
  int32_t start[JL_MAX_SEQS];  // first packed token of the sequence
  int32_t len[JL_MAX_SEQS];    // its length L_b
  int32_t G[JL_MAX_SEQS];      // its group size G_b
  int32_t vstart[JL_MAX_SEQS]; // first V^T column of the sequence (multiple of 64)
  int32_t vt_cols;             // V^T row length: sum of lengths rounded up to 64
};

// Work order of the bf16 prefill kernel (q tiles >= 1 of every sequence):
// sequences sorted by tile count c[] (descending), perm[] maps back.
struct JlSched {
  int32_t nlev;
  int32_t total_units;
  int32_t nxcd;                // XCDs of the device (workgroup n runs on XCD n % nxcd)
  int32_t xcd_heads;           // Hq / nxcd when Hq % nxcd == 0, else 0
  int32_t c[JL_MAX_SEQS];
  int32_t perm[JL_MAX_SEQS];
  uint8_t head_order[JL_MAX_HEADS];   // q heads grouped by kv head
};

// RoPE frequencies theta_m / (2 pi) in unsigned 0.64 fixed point (see
// jl_angle_turns in jl_mapper.h).
struct JlFreqs {
  uint64_t turn_frac[JL_MAX_HALF];
};

struct JlHeadMap {
  uint8_t kv_of[JL_MAX_HEADS];
  // with NG = Hq / Hkv q heads on every kv head: slot kvh * NG + n holds the
  // n-th q head (in head order) of kv head kvh (decode's head slots)
  uint8_t head_of_slot[JL_MAX_HEADS];
};

// Workspace of the prefill path: rotated operands, head-major.
//   qb, qr   [Hq][T_pad][d]   q rotated at p and at f(p) (fp32 path only; the
//            bf16 kernels rotate the caller's q rows themselves, and qb, qr
//            are null there)
//   kb, kr   [Hkv][T_pad][d]  k rotated at p and at f(p)
//   vt       [Hkv][vt_cols / 64][d][64] v transposed in 64-key tiles (bf16
//            path only); sequence b starts at key column vstart[b], a
//            multiple of 64, and its columns past L_b up to the next multiple
//            of 64 are zero
// Rows T .. T_pad-1 are zero.  qr / kr alias qb / kb when no sequence has
// G > 1.
//   kb_lo, kr_lo [Hkv][nseq * JL_LO_ROWS][d]
//            (bf16 path only) the rounding residuals bf16(x - bf16(x)) of the
//            first JL_LO_ROWS positions of every sequence, row b * JL_LO_ROWS + p
struct JlPrefillWs {
  void* qb;
  void* qr;
  void* kb;
  void* kr;
  void* vt;
  void* kb_lo;
  void* kr_lo;
  void* o1;      // [Hq][nseq * JL_LO_ROWS][d] fp32: normalised pass-1 output of the first rows
                 // (bf16 path, some G > 1; the 256-row kernel keeps its own in registers)
  void* o2;      // [Hq][T][d] fp32: normalised pass-2 output; the 256-row kernels keep each
                 // full 32-row group of a wave in that wave's lane order
  void* o3;      // [Hq][T][d] fp32: pass 3's accumulator of rows >= JL_LO_ROWS (scaled by
                 // exp2(-m3)), written and read back by the three-pass kernel; it is the o2
                 // array, whose rows >= JL_LO_ROWS only the disjoint variant uses otherwise
  void* lse1;    // [Hq][nseq * JL_LO_ROWS] fp32: pass-1 LogSumExp of the first rows, log2 units
  void* lse2;    // [Hq][T] fp32: pass-2 LogSumExp, log2 units
  void* ml3;     // [Hq][T] float2: pass 3's stabiliser m3 (log2 units) and sum l3, rows >= JL_LO_ROWS
  void* kc;      // [T][Hkv][d] dtype: base-rotated k in cache layout (optional output), or nullptr
  int64_t t_pad;
};

// Rows whose scores use split (hi + lo) bf16 operands: the first q tile of a
// sequence, whose rows see at most this many keys.
#define JL_LO_ROWS 128

// Shape of the device the calls launch on: compute units and XCDs (each XCD
// has its own L2; workgroup n of a dispatch runs on XCD n % xcds).  Read once
// per device (the library's only global state) from the current device; a
// host without a device gets the full MI355X shape, 256 CUs in 8 XCDs.
struct JlDevShape {
  int32_t cus;
  int32_t xcds;
};
JlDevShape jl_device_shape();

int64_t jl_prefill_t_pad(int64_t total_tokens);

// rope pre-pass: writes kb, kr and, for Hq > 0, qb, qr (elem = 2 for bf16, 4 for fp32; the bf16
// path passes Hq = 0); q is scaled by qscale
hipError_t jl_launch_rope_prepass(const void* q, const void* k, const JlPrefillWs& ws, int elem_bytes,
                                  int64_t total_tokens, int32_t Hq, int32_t Hkv, int32_t d,
                                  const JlSeqs& seqs, const JlFreqs& fr, float qscale, hipStream_t st);
// base RoPE of n rows [n][H][d] at positions pos0 .. pos0 + n - 1 (y may alias x)
hipError_t jl_launch_rope_rows(const void* x, void* y, int elem_bytes, int64_t n, int32_t H, int32_t d,
                               int64_t pos0, const JlFreqs& fr, hipStream_t st);
hipError_t jl_launch_transpose_v(const void* v, const JlPrefillWs& ws, const JlSeqs& seqs,
                                 int32_t Hkv, hipStream_t st);

hipError_t jl_launch_prefill_fp32(const JlPrefillWs& ws, const float* v, float* o, float* lse,
                                  int64_t total_tokens, int32_t Hq, int32_t Hkv, int32_t d,
                                  const JlHeadMap& hm, const JlSeqs& seqs, int64_t w0, float scale,
                                  int32_t max_len, hipStream_t st);

// disjoint: rows >= 128 merge pass 1 with a far-only pass (pairs i - j >= w0)
// instead of pass 2 minus pass 3
// q: the caller's [T][Hq][128] bf16 query, rotated by the kernels themselves
// (fr: the RoPE turn fractions; qscale: softmax scale * log2(e), folded into
// q before its bf16 rounding)
hipError_t jl_launch_prefill_bf16(const JlPrefillWs& ws, const void* q, const JlFreqs& fr, float qscale,
                                  void* o, float* lse, int64_t total_tokens, int32_t Hq, int32_t Hkv,
                                  const JlHeadMap& hm, const JlSeqs& seqs, int64_t w0, float scale,
                                  int32_t max_len, bool disjoint, hipStream_t st);

// decode: the sequences of one call, each with its own length, group size
// and cache rows; workgroup w serves sequence b for wg_begin[b] <= w <
// wg_begin[b + 1], keys [(w - wg_begin[b]) nsub 64, + nsub 64) of it
struct JlDecSeqs {
  int32_t nseq;
  int32_t nsub;                        // 64-key sub-chunks per workgroup (one value per call)
  int32_t wg_begin[JL_MAX_SEQS + 1];   // prefix sums of the workgroups per sequence; entries nseq .. JL_MAX_SEQS hold the total
  int32_t L[JL_MAX_SEQS];              // cached keys, the query at L - 1
  int32_t G[JL_MAX_SEQS];
  int32_t w0[JL_MAX_SEQS];             // window, L when every key is base (w0 >= L or G = 1)
  int64_t row0[JL_MAX_SEQS];           // first cache row of the sequence
  int64_t ws_wgs;                      // partial-result slots the workspace holds (>= the workgroups)
};
// plan of a call (host): nsub from the total key count, workgroups per sequence
// cus: compute units of the device (one split workgroup per compute unit)
void jl_decode_plan(const int64_t* lens, const int64_t* row0, int32_t nseq, int64_t w0,
                    int64_t w_pretrained, int32_t cus, JlDecSeqs* ds);
size_t jl_decode_workspace_bytes(const JlDecSeqs& ds, int32_t Hq);
hipError_t jl_launch_decode_bf16(const void* q, const void* k_cache, const void* v_cache,
                                 const JlDecSeqs& ds, void* o, float* lse, int32_t Hq, int32_t Hkv,
                                 const JlHeadMap& hm, float scale, const JlFreqs& fr, void* workspace,
                                 hipStream_t st);

// instrumentation: event to record after the dominant kernel, or nullptr
hipEvent_t jl_profile_mid_event();

// test hooks
hipError_t jl_launch_test_group_size(const int64_t* L, int64_t n, int64_t w, int64_t* G,
                                     hipStream_t st);
hipError_t jl_launch_test_remote_pos(int64_t x0, int64_t n, int32_t G, int32_t* f, hipStream_t st);
hipError_t jl_launch_test_angles(const int32_t* pos, int64_t n, uint64_t turn_frac, float* c,
                                 float* s, hipStream_t st);
// ceiling kernels (measurement): dense MFMA issue on every CU, streaming read
hipError_t jl_launch_mfma_peak(int64_t iters, float* sink, hipStream_t st);
hipError_t jl_launch_read_peak(const void* buf, int64_t bytes, int nt, float* sink, hipStream_t st);
