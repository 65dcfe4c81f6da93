// Correctly rounded float32 SiLU and SiLU' of bf16 inputs (device side).
//
// silu(u) = u / (1 + exp(-u)),  silu'(u) = s * (1 + u * (1 - s)), s = sigmoid(u),
// both rounded once to float32.  Evaluation:
//  * |u| in [2**-16, 2**8): a 6144-entry table per function, constant data of
//    the library written at build time (correctly rounded entries: float64
//    evaluation of the formula for |u| >= 2**-8, the series below under it),
//    staged through LDS by the kernels that use it;
//  * |u| >= 2**8: silu = u (u > 0) or -0 (u < 0); silu' = 1 or -0;
//  * |u| < 2**-16: the series u/2 + u**2/4 - u**4/48 (silu) and
//    1/2 + u/2 - u**3/12 (silu'): the float64 sum of the first two terms is
//    exact, and the next term only decides exact float32 midpoints (its sign).
#pragma once
#include "moe4_internal.h"

namespace moe4 {

constexpr int ACT_TAB = 6144;             // sign x 24 binades x 128 mantissas
constexpr uint32_t ACT_HALF = ACT_TAB / 2;  // entries per sign
constexpr uint32_t ACT_LO = 111u << 7;      // |bf16| bits of 2**-16, the first entry

// Offset of |u| in its sign's half of the table; ACT_HALF or more (unsigned
// wrap below 2**-16) when |u| is outside [2**-16, 2**8).
__device__ inline uint32_t act_slot(uint32_t b) { return (b & 0x7FFFu) - ACT_LO; }

// Table index of a bf16 pattern with |u| in [2**-16, 2**8), else -1.
__device__ inline int act_index(uint32_t b) {
  const uint32_t t = act_slot(b);
  if (t >= ACT_HALF) return -1;
  return (int)(t + (b >> 15) * ACT_HALF);
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

// The values of the patterns outside the table: |u| >= 2**8 by the limits,
// |u| < 2**8 (only ever below 2**-8 here) by the series.
template <bool DERIV>
__device__ inline float act_outside(uint32_t b) {
  float u = bf16_bits_to_f32(b);
  uint32_t ex = (b >> 7) & 0xFFu;
  if (ex > 134u) {  // |u| >= 256 (or non-finite, outside the contract)
    if (DERIV) return u > 0.0f ? 1.0f : -0.0f;
    return u > 0.0f ? u : -0.0f;
  }
  return DERIV ? dsilu_small(u) : silu_small(u);
}

// Evaluate from the bf16 bits, with `tab` the function's ACT_TAB-entry table
// (LDS or global).
template <bool DERIV>
__device__ inline float act_eval(uint32_t b, const float* tab) {
  const int idx = act_index(b);
  return idx >= 0 ? tab[idx] : act_outside<DERIV>(b);
}

// act_eval of the 2N bf16 patterns packed in w (low half first): when no lane
// of the wave holds a pattern outside the table (activations almost never
// reach below 2**-16 in magnitude), 2N plain table reads behind one
// wave-uniform test; otherwise act_eval for each.
template <bool DERIV, int N>
__device__ inline void act_eval_packed(const uint32_t (&w)[N], const float* tab, float (&out)[2 * N]) {
  bool outside = false;
#pragma unroll
  for (int i = 0; i < N; ++i) outside |= (act_slot(w[i] & 0xFFFFu) >= ACT_HALF) | (act_slot(w[i] >> 16) >= ACT_HALF);
  if (!__any(outside)) {
#pragma unroll
    for (int i = 0; i < 2 * N; ++i) {
      const uint32_t b = (i & 1) ? w[i >> 1] >> 16 : w[i >> 1] & 0xFFFFu;
      out[i] = tab[act_slot(b) + (b >> 15) * ACT_HALF];
    }
  } else {
#pragma unroll
    for (int i = 0; i < 2 * N; ++i)
      out[i] = act_eval<DERIV>((i & 1) ? w[i >> 1] >> 16 : w[i >> 1] & 0xFFFFu, tab);
  }
}

// Device address of the constant tables ([0] = silu, [1] = silu', ACT_TAB
// floats each) on the current device, in *out.  A symbol query, no stream
// work.  Returns 0 or an error code.
int act_tables(const float** out);

// Stage one table (ACT_TAB floats) into LDS; every thread of the block calls it.
__device__ inline void stage_act_table(float* lds, const float* gtab) {
  for (int i = threadIdx.x; i < ACT_TAB; i += blockDim.x) lds[i] = gtab[i];
  __syncthreads();
}

// The narrow table: the [2**-8, 2**8) part of a table (sign x 16 binades x 128
// mantissas), 16 KB of LDS for kernels with little LDS to spare, read through
// act_eval_narrow (the series below 2**-8).
constexpr int ACT_NARROW = 4096;
constexpr uint32_t ACT_NARROW_LO = 119u << 7;  // |bf16| bits of 2**-8

__device__ inline void stage_act_table_narrow(float* lds, const float* gtab) {
  constexpr uint32_t skip = ACT_NARROW_LO - ACT_LO;  // entries below 2**-8 in each half of the full table
  for (int i = threadIdx.x; i < ACT_NARROW; i += blockDim.x) lds[i] = gtab[(i >> 11) * ACT_HALF + skip + (i & 2047)];
  __syncthreads();
}

template <bool DERIV>
__device__ inline float act_eval_narrow(uint32_t b, const float* ntab) {
  const uint32_t t = (b & 0x7FFFu) - ACT_NARROW_LO;
  return t < 2048u ? ntab[t + ((b >> 15) << 11)] : act_outside<DERIV>(b);
}

}  // namespace moe4
