/*
 * jetlong_testing.h - test-only entry points of libjetlong.so.
 *
 * They expose the DEVICE build of the position mapper so that tests can
 * check it bit for bit against exact integer arithmetic (technical summary
 * on gist.science, Methodology item 1: group-size equation
 * G = max(1, ceil(L / w_pretrained)) and remote map f(x) = floor(x / G)).
 * They are not part of the attention path.  Pointers are device memory owned
 * by the caller; launches are asynchronous on `hip_stream`.
 */
#ifndef JETLONG_TESTING_H
#define JETLONG_TESTING_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* G_out[i] = G(L[i], w_pretrained) computed on the device, i < n.
   JL_EINVAL if n < 0, w_pretrained < 1 or a pointer is NULL with n > 0.
   Negative L[i] produce G_out[i] = -1. */
int jl_test_group_size_device(const int64_t* L, int64_t n, int64_t w_pretrained, int64_t* G_out,
                              void* hip_stream);

/* f_out[i] = f(x0 + i) = floor((x0 + i) / G) computed on the device with the
   same 32-bit routine the kernels use, i < n.  Requires 0 <= x0,
   x0 + n <= 2^31 - 1, G >= 1. */
int jl_test_remote_pos_device(int64_t x0, int64_t n, int64_t G, int32_t* f_out, void* hip_stream);

/* cos_out[i], sin_out[i] = cos / sin of the angle pos[i] * theta_m (theta_m =
   rope_base^(-2m/head_dim)) as the kernels form it (fixed-point revolutions,
   then fp32 sin/cos), i < n.  Lets tests bound the angle error at long
   positions. */
int jl_test_rope_angles_device(const int32_t* pos, int64_t n, int32_t m, int32_t head_dim,
                               double rope_base, float* cos_out, float* sin_out, void* hip_stream);

/* Instrumentation for benchmarks: while set, every prefill and decode call
   (jl_bifocal_prefill, jl_bifocal_prefill_disjoint, jl_bifocal_decode,
   jl_bifocal_decode_batch) made on the calling thread records hipEvent_t
   `before` on its stream immediately before launching its attention
   kernels, `mid` (optional, may be NULL) right after its dominant kernel
   (prefill: the full-causal pass-2 launches, or the far pass of the
   disjoint form; decode: the split-K launch), and `after` after the last of
   them.  The RoPE pre-pass of prefill stays
   outside.  Pass NULL for all three to stop.  The events are the caller's;
   the library never creates or destroys them.  Returns JL_EINVAL if exactly
   one of `before` and `after` is NULL. */
int jl_set_profile_events(void* before, void* mid, void* after);

/* The device shape the library plans with: compute units and XCDs of the
   current device, read once per device (hipDeviceAttributeMultiprocessorCount
   and hipDeviceAttributeNumberOfXccs).  A host without a device reports the
   full MI355X shape, 256 and 8.  Host function. */
int jl_test_device_shape(int32_t* cus, int32_t* xcds);

/* The decode plan (host function, nothing launched) for num_seqs sequences
   of lens[b] keys on a device with `cus` compute units: *nsub = 64-key
   sub-chunks per split workgroup, *nwg = split workgroups.  The plan takes
   the smallest nsub whose workgroups fit one round (one per compute unit).
   JL_EINVAL on a NULL pointer, cus < 1, num_seqs outside 1 .. JL_MAX_SEQS or
   a length outside 0 .. 2^31 - 1. */
int jl_test_decode_plan(const int64_t* lens, int32_t num_seqs, int32_t cus, int32_t* nsub, int32_t* nwg);

/* The same plan's workgroup prefix sums: wg_begin[b] = first split workgroup
   of sequence b, for b = 0 .. JL_MAX_SEQS (JL_MAX_SEQS + 1 entries, written
   by the call).  The decode kernels rely on two properties of it: the entries
   never decrease (a workgroup finds its sequence by counting the starts at
   or before it), and every entry from num_seqs on holds the total workgroup
   count (read at a fixed offset).  Same errors as jl_test_decode_plan. */
int jl_test_decode_prefix(const int64_t* lens, int32_t num_seqs, int32_t cus, int32_t* wg_begin);

/* Ceiling kernels for benchmarks: what the chip achieves on its own, the
   denominators beside the published peaks.
   jl_bench_mfma_peak: one workgroup of 8 waves per compute unit, each wave
   issuing iters x 32 dense v_mfma_f32_32x32x16_bf16 in four independent
   accumulator chains and nothing else; *flops receives the FLOPs of the
   launch.  jl_bench_read_peak: a streaming read of `bytes` (a multiple of 16,
   16-byte aligned device memory) with 16-byte loads, default or
   non-temporal cache policy, each workgroup (one per compute unit) streaming
   its own contiguous share with eight 16-byte loads in flight per thread.
   sink: one device float, written only under a
   condition the kernels never meet.  Asynchronous on hip_stream; the caller
   times them.  JL_EINVAL on bad arguments. */
int jl_bench_mfma_peak(int64_t iters, float* sink, int64_t* flops, void* hip_stream);
int jl_bench_read_peak(const void* buf, int64_t bytes, int32_t nontemporal, float* sink, void* hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* JETLONG_TESTING_H */
