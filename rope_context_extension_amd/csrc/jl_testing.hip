// jl_testing.hip - kernels behind the test-only entry points: they run the
// device build of the position mapper and of the angle formation
// (jl_mapper.h) over caller-provided ranges.
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
