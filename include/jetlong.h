/*
 * jetlong.h - C ABI of the MI355X (gfx950) bifocal RoPE attention library.
 *
 * Jet-Long ("Jet-Long: Efficient Long-Context Extension with Dynamic Bifocal
 * RoPE") extends a RoPE model past its pretraining window without training.
 * Every (query i, key j) score of causal attention is routed by distance:
 *   - pairs with i - j < w0 use ordinary RoPE at the absolute positions i, j;
 *   - farther pairs use RoPE at the aliased positions f(i), f(j),
 *     f(x) = floor(x / G), G = max(1, ceil(L / w_pretrained)).
 * (technical summary on gist.science, Methodology item 1, "Dynamic Bifocal
 * RoPE": local window, remote window, group-size equation and remote map).
 *
 * Conventions shared by every entry point:
 *   - Tensor pointers are DEVICE memory owned by the caller.  The library
 *     never allocates or frees device memory and keeps no pointer after a
 *     call returns.  Scratch space is the caller's `workspace` (two-call
 *     protocol: pass workspace == NULL to get the size in *workspace_bytes;
 *     nothing is launched then).
 *   - Host pointers (q_to_kv, cu_seqlens) are read during the call only.
 *   - `hip_stream` is a hipStream_t passed as void* (NULL = default stream).
 *     Launches are asynchronous on that stream; the caller synchronises.
 *   - Every argument is validated before anything is launched: a JL_EINVAL
 *     or JL_EUNSUPPORTED return has no side effect.  A failed launch returns
 *     JL_EHIP.  jl_last_error() gives a message for the calling thread.
 *   - Empty work (zero tokens, L == 0) returns JL_OK and launches nothing.
 *   - Layouts are row-major and contiguous.  RoPE pairs dimension m with
 *     m + d/2 and uses theta_m = rope_base^(-2m/d) (the rotary layout of the
 *     Qwen3 models the pages evaluate).  Angles are exact: theta_m / 2pi is
 *     reduced mod 1 on the host into a 0.64 fixed-point fraction of a turn,
 *     the device multiplies it by the integer position mod 2^64, and only
 *     the remaining fraction of a turn goes through fp32 sin/cos.
 *   - softmax_scale <= 0 selects 1/sqrt(head_dim).  LSE outputs are the
 *     natural log of sum_j exp(softmax_scale * q.k) per (head, row), fp32.
 *   - q_to_kv: host int32[num_q_heads] giving the kv head of each q head, or
 *     NULL for h / (num_q_heads / num_kv_heads).
 */
#ifndef JETLONG_H
#define JETLONG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  JL_OK = 0,
  JL_EINVAL = -1,        /* an argument is out of its documented range */
  JL_EUNSUPPORTED = -2,  /* valid, but not built (dtype, head_dim, sizes) */
  JL_ENOSPC = -3,        /* *workspace_bytes is smaller than required */
  JL_EHIP = -4           /* a HIP launch or runtime call failed */
} jl_status;

typedef enum { JL_BF16 = 0, JL_FP32 = 1 } jl_dtype;

/* Largest number of sequences one jl_bifocal_prefill or jl_bifocal_decode_batch call accepts. */
#define JL_MAX_SEQS 64

/* Longest sequence the bf16 prefill accepts, 2^23 - 64 tokens: its tile copies address a sequence's
   K and V rows (256 bytes per key) with 31-bit byte offsets. */
#define JL_BF16_MAX_SEQ_LEN 8388544

/* Longest sequence the fp32 prefill accepts, 2^24 tokens: it runs one 64-lane workgroup per query row,
   and one dispatch holds fewer than 2^32 work-items. */
#define JL_FP32_MAX_SEQ_LEN 16777216

/*
 * Group size G = max(1, ceil(L / w_pretrained)) (technical summary,
 * Methodology item 1, group-size equation).  Host integer function, exact
 * for all int64 inputs.  Returns G >= 1, or JL_EINVAL (< 0) if L < 0 or
 * w_pretrained < 1.
 */
int64_t jl_group_size(int64_t L, int64_t w_pretrained);

/*
 * Bifocal causal prefill over packed independent sequences, computed as the
 * inclusion-exclusion merge of three flash passes combined through their
 * LogSumExp statistics (technical summary, Methodology item 2, "Inference
 * efficiency mechanisms": local window with base q/k, full causal with
 * remote q/k, local window with remote q/k; no mask matrix).  With
 * lse_k = log sum of pass k's weights, M = max(lse_1, lse_2) and
 * z_k = exp(lse_k - M), the far mass z2 - z3 is clamped at zero:
 *   far = max(z2 - z3, 0),
 *   out = (z1 o1 + [far > 0] (z2 o2 - z3 o3)) / (z1 + far),
 *   lse = M + log(z1 + far).
 * In exact arithmetic z2 >= z3 and the clamp changes nothing; it keeps the
 * result finite when rounding makes the difference negative.  With JL_BF16,
 * rows from the 129th of a sequence on take passes 2 and 3 from one walk over
 * the remote-grid key tiles (the state after the window tiles is pass 3's),
 * and z2 o2 - z3 o3 and z2 - z3 are formed from the two states' accumulators,
 * maxima and sums in the frame of pass 2's maximum, which is the same
 * quantity.  Precision: the far mass is the difference of two
 * window-dominated terms, so a row whose far mass is small against its
 * window mass under the remote grid, yet comparable to the base-grid window
 * mass, loses relative precision in that term (fp32 rounding of the window
 * terms times their ratio to the far mass).  With q, k ~ N(0, 25) this can
 * move the output outside the range of V.  jl_bifocal_prefill_disjoint
 * computes the same attention with two positive weights and no cancelling
 * term; prefer it for such inputs.
 *
 *   q          [total_tokens, num_q_heads, head_dim]  raw (pre-RoPE), dtype
 *   k, v       [total_tokens, num_kv_heads, head_dim] raw (pre-RoPE), dtype
 *   o          [total_tokens, num_q_heads, head_dim]  dtype (written)
 *   lse        [num_q_heads, total_tokens] fp32, or NULL
 *   cu_seqlens host int64[num_seqs + 1], cu_seqlens[0] = 0, non-decreasing,
 *              cu_seqlens[num_seqs] = total_tokens; NULL means one sequence
 *              of total_tokens.  Positions restart at 0 in every sequence and
 *              each sequence uses its own G from its own length.
 *   num_seqs   1 .. JL_MAX_SEQS
 *   head_dim   64 or 128 (JL_BF16 needs 128; JL_FP32 accepts both)
 *   dtype      JL_BF16: bf16 MFMA passes with fp32 accumulation, bf16 o.
 *              JL_FP32: fp32 vector-ALU passes (exactness reference path).
 *   w0         >= 0 local window; w_pretrained >= 1; rope_base > 0.
 *   With JL_BF16, sequences longer than JL_BF16_MAX_SEQ_LEN tokens are
 *   JL_EUNSUPPORTED; with JL_FP32, longer than JL_FP32_MAX_SEQ_LEN.  Either
 *   way total_tokens is at most 2^31 - 513.
 *   The work order follows the current device's XCD count (it must be the
 *   device of hip_stream); results do not depend on it.
 */
int jl_bifocal_prefill(const void* q, const void* k, const void* v, void* o, float* lse,
                       const int64_t* cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                       int32_t num_q_heads, int32_t num_kv_heads, const int32_t* q_to_kv,
                       int32_t head_dim, jl_dtype dtype, int64_t w0, int64_t w_pretrained,
                       double rope_base, float softmax_scale, void* workspace,
                       size_t* workspace_bytes, void* hip_stream);

/*
 * jl_bifocal_prefill that also writes the decode cache of its keys
 * (technical summary, Methodology item 2: the cache holds the keys rotated by
 * base RoPE at their absolute positions, and generation continues from it
 * without rewriting it).  The pre-pass that rotates k for the attention
 * passes also stores the base-rotated key of every token in the input's
 * layout, so a prefill followed by decode steps needs no second pass over k:
 *
 *   k_cache    [total_tokens, num_kv_heads, head_dim] dtype (written),
 *              16-byte aligned, overlapping none of q, k, v, o, lse or the
 *              workspace.  Row t of sequence b (t = cu_seqlens[b] + p) holds
 *              k[t] rotated at position p of that sequence, the same bits
 *              jl_rope_rows writes for those rows at pos0 = 0.
 *
 * Every other argument, the workspace size, o, lse and the errors are those
 * of jl_bifocal_prefill (o and lse are bitwise its results); a size query
 * (workspace NULL) ignores k_cache, and a call with a workspace and
 * total_tokens > 0 needs k_cache non-NULL (JL_EINVAL).
 */
int jl_bifocal_prefill_kcache(const void* q, const void* k, const void* v, void* o, float* lse,
                              void* k_cache, const int64_t* cu_seqlens, int32_t num_seqs,
                              int64_t total_tokens, int32_t num_q_heads, int32_t num_kv_heads,
                              const int32_t* q_to_kv, int32_t head_dim, jl_dtype dtype, int64_t w0,
                              int64_t w_pretrained, double rope_base, float softmax_scale,
                              void* workspace, size_t* workspace_bytes, void* hip_stream);

/*
 * The same bifocal prefill with the far pairs computed directly instead of as
 * a difference of two passes (technical summary, Methodology item 2: pairs
 * inside the local window see base-RoPE q/k, all farther pairs see the
 * remote grid).  Rows >= 128 of every sequence run the window pass on the
 * base grid and one pass over the pairs with i - j >= w0 on the remote grid,
 * merged as out = (z1 o1 + zf of) / (z1 + zf): both weights are positive, so
 * no term cancels (the three-pass form subtracts z3 o3 from z2 o2, which
 * loses relative precision where the far mass is small against the window
 * mass).  Rows < 128 of a sequence take the three-pass path.
 *
 * Arguments, layouts, workspace size (query it through jl_bifocal_prefill or
 * this call: they are equal) and errors are those of jl_bifocal_prefill;
 * JL_FP32 is JL_EUNSUPPORTED here.
 */
int jl_bifocal_prefill_disjoint(const void* q, const void* k, const void* v, void* o, float* lse,
                                const int64_t* cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                                int32_t num_q_heads, int32_t num_kv_heads, const int32_t* q_to_kv,
                                int32_t head_dim, jl_dtype dtype, int64_t w0, int64_t w_pretrained,
                                double rope_base, float softmax_scale, void* workspace,
                                size_t* workspace_bytes, void* hip_stream);

/*
 * One single-batch generation step against a KV cache of base-RoPE keys
 * (technical summary, Methodology item 2: the cache holds uncompressed base
 * keys at their absolute positions; the correction rotation Delta is applied
 * to the active query and the cached keys on the fly, and the cache is never
 * rewritten, also when L crosses a G boundary).
 *
 *   q        [num_q_heads, head_dim] bf16, already rotated by base RoPE at
 *            position L - 1 (the query of the newest token)
 *   k_cache  [L_cap, num_kv_heads, head_dim] bf16; row j holds the key
 *            rotated at absolute position j; rows 0 .. L-1 are valid (the
 *            current token's key included).  Read only.
 *   v_cache  [L_cap, num_kv_heads, head_dim] bf16.  Read only.
 *   L        number of valid cache rows, 0 .. 2^31 - 1; G = jl_group_size(L).
 *            Keys with (L - 1) - j < w0 score with the base vectors; the rest
 *            score with R(f(L-1) - (L-1)) q and R(f(j) - j) k_j.
 *   o        [num_q_heads, head_dim] bf16 (written)
 *   lse      [num_q_heads] fp32, or NULL
 *   head_dim 128; dtype must be JL_BF16.
 *   The split of the keys over workgroups (and so the workspace size) follows
 *   the compute-unit count of the current device, which must be the device
 *   of hip_stream: query the size and call with the same device current.
 *   The workspace size never decreases as L grows, so a workspace sized for
 *   the longest step of a generation loop serves every shorter step.
 */
int jl_bifocal_decode(const void* q, const void* k_cache, const void* v_cache, int64_t L,
                      void* o, float* lse, int32_t num_q_heads, int32_t num_kv_heads,
                      const int32_t* q_to_kv, int32_t head_dim, jl_dtype dtype, int64_t w0,
                      int64_t w_pretrained, double rope_base, float softmax_scale,
                      void* workspace, size_t* workspace_bytes, void* hip_stream);

/*
 * One generation step for each of num_seqs independent sequences with their
 * own lengths (ragged), in one call: sequence b is exactly jl_bifocal_decode
 * with L = lens[b], its own G = jl_group_size(lens[b]) and its own query
 * (technical summary, Methodology item 2, applied per sequence: every
 * sequence keeps its base-RoPE cache rows and gets its own correction
 * rotation; the pages measure one sequence only).
 *
 *   q          [num_seqs, num_q_heads, head_dim] bf16; q[b] is rotated by base
 *              RoPE at position lens[b] - 1
 *   k_cache, v_cache  [cache_rows, num_kv_heads, head_dim] bf16, read only;
 *              sequence b's key j (rotated at absolute position j) is row
 *              row0[b] + j.  Ranges of different sequences may overlap.
 *   row0, lens host int64[num_seqs]: row0[b] >= 0, 0 <= lens[b] < 2^31,
 *              row0[b] + lens[b] <= cache_rows (else JL_EINVAL)
 *   num_seqs   1 .. JL_MAX_SEQS
 *   o          [num_seqs, num_q_heads, head_dim] bf16 (written)
 *   lse        [num_seqs, num_q_heads] fp32, or NULL
 *   Sequences with lens[b] == 0 are skipped: their o rows and lse entries
 *   are not written.  Workspace: two-call protocol as in jl_bifocal_decode;
 *   its size depends on lens and never decreases as any lens[b] grows.  The
 *   other arguments and errors are those of jl_bifocal_decode.
 */
int jl_bifocal_decode_batch(const void* q, const void* k_cache, const void* v_cache, int64_t cache_rows,
                            const int64_t* row0, const int64_t* lens, int32_t num_seqs, void* o,
                            float* lse, int32_t num_q_heads, int32_t num_kv_heads,
                            const int32_t* q_to_kv, int32_t head_dim, jl_dtype dtype, int64_t w0,
                            int64_t w_pretrained, double rope_base, float softmax_scale,
                            void* workspace, size_t* workspace_bytes, void* hip_stream);

/*
 * Base RoPE of n consecutive rows: y[r][h][:] = R(pos0 + r) x[r][h][:],
 * half-split pairs (m, m + head_dim/2) at theta_m = rope_base^(-2m/head_dim),
 * with the same angle arithmetic as the prefill's base grid.  It builds or
 * extends the decode cache of keys rotated at their absolute positions and
 * rotates the newest query (technical summary, Methodology item 2: the cache
 * holds base keys; the correction rotation is decode's own business).
 *
 *   x, y       [n_rows, num_heads, head_dim] dtype, device; y may equal x
 *              (in place), otherwise the ranges must not overlap
 *   pos0       position of row 0, >= 0; pos0 + n_rows - 1 < 2^31 (so any
 *              n_rows up to 2^31 is launched, in a grid-stride loop)
 *   head_dim   even, <= 128
 *   n_rows == 0 does nothing.
 */
int jl_rope_rows(const void* x, void* y, int64_t n_rows, int32_t num_heads, int32_t head_dim,
                 jl_dtype dtype, int64_t pos0, double rope_base, void* hip_stream);

/* Bytes of the device scratch that jl_bifocal_decode_noalloc uses for its split-K partial results:
   256 split workgroups x 32 q heads x (max, sum, 128 channels) fp32. */
#define JL_DECODE_SCRATCH_BYTES 4259840

/*
 * jl_bifocal_decode without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, serving loops, hosts
 * that forbid allocation): the split-K partial results go to a scratch array
 * of JL_DECODE_SCRATCH_BYTES that the library holds in device memory (one
 * per GPU, kept until the process ends; its address is looked up once per
 * device).  Nothing is allocated and no allocating routine is called.
 *
 * Arguments, layouts, results and errors are those of jl_bifocal_decode (the
 * same kernels and the same split, so the outputs are bitwise those of
 * jl_bifocal_decode).  A call whose partials exceed the scratch
 * (jl_bifocal_decode's workspace size for the same arguments above
 * JL_DECODE_SCRATCH_BYTES; e.g. more than 32 q heads on a 256-CU device) is
 * JL_EUNSUPPORTED before anything is launched.  Every call on one GPU shares
 * that GPU's scratch, so calls that overlap in time on one GPU (different
 * streams, or different host threads without ordering) race; calls ordered
 * on one stream do not.
 */
int jl_bifocal_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, int64_t L,
                              void* o, float* lse, int32_t num_q_heads, int32_t num_kv_heads,
                              const int32_t* q_to_kv, int32_t head_dim, jl_dtype dtype, int64_t w0,
                              int64_t w_pretrained, double rope_base, float softmax_scale, void* hip_stream);

/* Message describing the last non-JL_OK return on the calling thread. */
const char* jl_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* JETLONG_H */
