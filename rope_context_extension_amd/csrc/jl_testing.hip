// jl_testing.hip - kernels behind the test-only entry points: they run the
// device build of the position mapper and of the angle formation
// (jl_mapper.h) over caller-provided ranges, and two ceiling kernels that
// measure what the chip achieves on its own (dense bf16 MFMA issue, streaming
// HBM reads), the denominators beside the published peaks.
#include "jl_internal.h"

namespace {

__global__ void group_size_kernel(const int64_t* L, int64_t n, int64_t w, int64_t* G) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) G[i] = L[i] < 0 ? -1 : jl_group_size_i64(L[i], w);
}

__global__ void remote_pos_kernel(int64_t x0, int64_t n, int32_t G, int32_t* f) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) f[i] = jl_remote_pos((int32_t)(x0 + i), G);
}

__global__ void angles_kernel(const int32_t* pos, int64_t n, uint64_t tf, float* c, float* s) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) jl_rope_sincos(pos[i], tf, &s[i], &c[i]);
}

unsigned blocks(int64_t n) { return (unsigned)((n + 255) / 256); }

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Dense bf16 MFMA issue with nothing else: 8 waves (two per SIMD), each with
// four independent 32x32x16 accumulator chains, iters x 32 MFMAs per wave.
// The result goes to *sink only if it equals a value it never takes, which
// keeps the work from being removed.
__global__ void __launch_bounds__(512, 1) mfma_peak_kernel(int64_t iters, float* sink) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(lane * 0.01f + i);
    b[i] = (__bf16)(i * 0.5f);
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
    }
  }
  float r = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) r += c0[i] + c1[i] + c2[i] + c3[i];
  if (r == -1.2345e-30f) sink[0] = r;
}

// Streaming read: workgroup b reads its own contiguous share of the buffer
// with 16-byte loads, eight in flight per thread (the access pattern of the
// decode split, where each workgroup streams its own key range).  NT:
// non-temporal loads.
template <bool NT>
__device__ inline u32x4 ld16(const u32x4* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}

template <bool NT>
__global__ void __launch_bounds__(256) read_peak_kernel(const u32x4* __restrict__ buf, int64_t n16, float* sink) {
  const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const int64_t lo = (int64_t)blockIdx.x * per;
  const int64_t hi = lo + per < n16 ? lo + per : n16;
  uint32_t acc = 0;
  for (int64_t i = lo + threadIdx.x; i < hi; i += 256 * 8) {
    u32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = i + u * 256 < hi ? ld16<NT>(buf + i + u * 256) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (acc == 0x9e3779b9u && n16 < 0) sink[0] = (float)acc;
}

}  // namespace

hipError_t jl_launch_test_group_size(const int64_t* L, int64_t n, int64_t w, int64_t* G, hipStream_t st) {
  group_size_kernel<<<blocks(n), 256, 0, st>>>(L, n, w, G);
  return hipGetLastError();
}

hipError_t jl_launch_test_remote_pos(int64_t x0, int64_t n, int32_t G, int32_t* f, hipStream_t st) {
  remote_pos_kernel<<<blocks(n), 256, 0, st>>>(x0, n, G, f);
  return hipGetLastError();
}

hipError_t jl_launch_test_angles(const int32_t* pos, int64_t n, uint64_t turn_frac, float* c, float* s,
                                 hipStream_t st) {
  angles_kernel<<<blocks(n), 256, 0, st>>>(pos, n, turn_frac, c, s);
  return hipGetLastError();
}

hipError_t jl_launch_mfma_peak(int64_t iters, float* sink, hipStream_t st) {
  mfma_peak_kernel<<<(unsigned)jl_device_shape().cus, 512, 0, st>>>(iters, sink);
  return hipGetLastError();
}

hipError_t jl_launch_read_peak(const void* buf, int64_t bytes, int nt, float* sink, hipStream_t st) {
  const unsigned grid = (unsigned)jl_device_shape().cus;   // one workgroup per compute unit
  if (nt) read_peak_kernel<true><<<grid, 256, 0, st>>>((const u32x4*)buf, bytes / 16, sink);
  else read_peak_kernel<false><<<grid, 256, 0, st>>>((const u32x4*)buf, bytes / 16, sink);
  return hipGetLastError();
}
