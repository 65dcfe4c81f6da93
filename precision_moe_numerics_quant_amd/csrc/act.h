// Correctly rounded float32 SiLU and SiLU' of bf16 inputs (device side).
//
// silu(u) = u / (1 + exp(-u)),  silu'(u) = s * (1 + u * (1 - s)), s = sigmoid(u),
// both rounded once to float32.  Evaluation:
//  * |u| in [2**-8, 2**8): a 4096-entry table per function, constant data of
//    the library written at build time by evaluating the formula in float64
//    (whose error, ~1e-16, is far below the distance of every such entry from
//    a float32 rounding boundary), staged through LDS by the kernels that use
//    it;
//  * |u| >= 2**8: silu = u (u > 0) or -0 (u < 0); silu' = 1 or -0;
//  * |u| < 2**-8: the series u/2 + u**2/4 - u**4/48 (silu) and
//    1/2 + u/2 - u**3/12 (silu'): the float64 sum of the first two terms is
//    exact, and the next term only decides exact float32 midpoints (its sign).
#pragma once
#include "moe4_internal.h"

namespace moe4 {

constexpr int ACT_TAB = 4096;  // sign x 16 binades x 128 mantissas

// Table index of a bf16 pattern with |u| in [2**-8, 2**8), else -1.
__device__ inline int act_index(uint32_t b) {
  uint32_t ex = (b >> 7) & 0xFFu;
  if (ex < 119u || ex > 134u) return -1;
  return (int)(((b >> 15) << 11) | ((ex - 119u) << 7) | (b & 0x7Fu));
}

// Neighbouring float32 of a finite r, upward (up) or downward.
__device__ inline float next_float(float r, bool up) {
  uint32_t b = __float_as_uint(r);
  if ((b & 0x7FFFFFFFu) == 0u) return __uint_as_float(up ? 1u : 0x80000001u);
  const bool neg = (b >> 31) != 0u;
  return __uint_as_float((up != neg) ? b + 1u : b - 1u);
}

// Round a float64 value to float32; an exact float32 midpoint goes toward
// `dir` (-1: down, +1: up).
__device__ inline float round_dir(double a, int dir) {
  float r = (float)a;
  double d = a - (double)r;
  if (d == 0.0) return r;
  float n = next_float(r, d > 0);
  if ((double)n - a == d) return dir < 0 ? fminf(r, n) : fmaxf(r, n);  // a is the midpoint of r and n
  return r;
}

__device__ inline float silu_small(float u) {
  if (u == 0.0f) return u;
  double x = u;
  return round_dir(0.5 * x + 0.25 * (x * x), -1);
}

__device__ inline float dsilu_small(float u) {
  double x = u;
  return round_dir(0.5 + 0.5 * x, u > 0.0f ? -1 : 1);
}

// Evaluate from the bf16 bits, with `tab` the function's 4096-entry table
// (LDS or global).
template <bool DERIV>
__device__ inline float act_eval(uint32_t b, const float* tab) {
  int idx = act_index(b);
  if (idx >= 0) return tab[idx];
  float u = bf16_bits_to_f32(b);
  uint32_t ex = (b >> 7) & 0xFFu;
  if (ex > 134u) {  // |u| >= 256 (or non-finite, outside the contract)
    if (DERIV) return u > 0.0f ? 1.0f : -0.0f;
    return u > 0.0f ? u : -0.0f;
  }
  return DERIV ? dsilu_small(u) : silu_small(u);
}

// Device address of the constant tables ([0] = silu, [1] = silu', ACT_TAB
// floats each) on the current device, in *out.  A symbol query, no stream
// work.  Returns 0 or an error code.
int act_tables(const float** out);

// Stage one table (4096 floats) into LDS; every thread of the block calls it.
__device__ inline void stage_act_table(float* lds, const float* gtab) {
  for (int i = threadIdx.x; i < ACT_TAB; i += blockDim.x) lds[i] = gtab[i];
  __syncthreads();
}

}  // namespace moe4
