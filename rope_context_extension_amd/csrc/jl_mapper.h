// jl_mapper.h - position mapper and RoPE angle formation, host and device.
//
// Group size and remote map: technical summary on gist.science, Methodology
// item 1 ("Dynamic Bifocal RoPE"): G = max(1, ceil(L / w_pretrained)) and
// f(x) = floor(x / G).  The same inline code is compiled for the host (the
// C ABI, argument validation, scheduling) and for gfx950 (the kernels).
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define JL_HD __host__ __device__ inline
#else
#define JL_HD inline
#endif

// ceil(L / w) for L >= 1 written as (L - 1) / w + 1 so no intermediate can
// overflow int64; L == 0 gives the max(1, .) floor value 1.  Callers check
// w >= 1 and L >= 0.
JL_HD int64_t jl_group_size_i64(int64_t L, int64_t w_pretrained) {
  return L <= 0 ? 1 : (L - 1) / w_pretrained + 1;
}

// f(x) = floor(x / G) for 0 <= x < 2^31 (C division truncates, which is the
// floor for non-negative operands).
JL_HD int32_t jl_remote_pos(int32_t x, int32_t G) { return x / G; }

// RoPE angle of integer position p for frequency theta_m, as a fraction of a
// full turn.  `turn_frac` is theta_m / (2 pi) in unsigned 0.64 fixed point
// (built on the host in extended precision).  The product p * turn_frac
// wraps modulo 2^64, which is exactly the reduction of the angle modulo one
// turn, so the reduction adds no error however large |p| is; only the
// fixed-point rounding of theta_m / (2 pi) (2^-64 relative) scales with p.
// The top 32 bits, read as a signed fraction of a turn in [-1/2, 1/2), are
// then handed to an fp32 sin/cos of pi * y with y in [-1, 1).
JL_HD uint64_t jl_angle_turns(int32_t p, uint64_t turn_frac) {
  return (uint64_t)(int64_t)p * turn_frac;
}

#if defined(__HIPCC__)
__device__ inline void jl_rope_sincos(int32_t p, uint64_t turn_frac, float* s, float* c) {
  const int32_t hi = (int32_t)(jl_angle_turns(p, turn_frac) >> 32);
  const float y = (float)hi * (1.0f / 2147483648.0f);   // angle = pi * hi / 2^31
  sincospif(y, s, c);
}

// The rotation of one half-split pair (x1, x2) = (x[m], x[m + d/2]) by
// (c, s) = (cos, sin) of its angle, with its fused multiply-adds written out:
// every kernel that rotates the same input at the same position (the RoPE
// pre-pass, the row rotation, the prefill kernels' query rotation) gets the
// same bits.
__device__ inline void jl_rot_pair(float x1, float x2, float c, float s, float* y1, float* y2) {
  *y1 = __builtin_fmaf(x1, c, -(x2 * s));
  *y2 = __builtin_fmaf(x2, c, x1 * s);
}
#endif
