// NVFP4 block encoding shared by the quantiser kernels (device code only):
// the E4M3 block scale of one candidate and the E2M1 codes it gives.
#pragma once
#include "moe4_internal.h"

namespace moe4 {

// E4M3 code (RNE, clamp to 448) of a non-negative finite float.
__device__ inline uint32_t e4m3_rne_u(float u) {
  u = fminf(u, 448.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(u, 0.0f, 0, false) & 0xFFu;
}

struct Cand {
  uint32_t sc;      // E4M3 scale byte
  uint32_t q[2];    // 16 packed nibbles
  float err;
};

// One candidate of one 16-block (steps: scale, encode, dequantise, error).
__device__ inline Cand encode_candidate(const float* x, float amax_b, float S, float m) {
  Cand c;
  const float d = m * S;
  const float u = amax_b / d;
  c.sc = e4m3_rne_u(u);
  const float scf = e4m3_to_f32(c.sc);
  const float eff = scf * S;
  const bool zero = (c.sc == 0u) || (eff == 0.0f);
  if (zero) {
    // every code a signed zero: deq = 0, t = x
    uint32_t q0 = 0, q1 = 0;
    float err = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      uint32_t sgn = (__float_as_uint(x[i]) >> 31) << 3;
      if (i < 8) q0 |= sgn << (4 * i); else q1 |= sgn << (4 * (i - 8));
      float t = x[i];
      err = err + t * t;
    }
    c.q[0] = q0; c.q[1] = q1; c.err = err;
    return c;
  }
  const float inv = 1.0f / eff;
  const bool inv_inf = __builtin_isinf(inv);
  const float mant = mant_factor(scf);
  uint32_t q0 = 0, q1 = 0;
  float err = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; i += 2) {
    float y0 = x[i] * inv, y1 = x[i + 1] * inv;
    if (inv_inf) {  // 0 * inf: a zero element stays a signed zero
      if (x[i] == 0.0f) y0 = x[i];
      if (x[i + 1] == 0.0f) y1 = x[i + 1];
    }
    // E2M1, round to nearest even, saturating, sign kept (scale 1: no rescale)
    uint32_t pk = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, y0, y1, 1.0f, 0) & 0xFFu;
    if (i < 8) q0 |= pk << (4 * i); else q1 |= pk << (4 * (i - 8));
    // exact q * 2**floor(log2 sc), times the mantissa 1.m: the exact q * sc
    f32x2 p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(pk, scf, 0);
    float p0 = p[0] * mant, p1 = p[1] * mant;
    float t0 = x[i] - p0 * S;
    float t1 = x[i + 1] - p1 * S;
    err = err + t0 * t0;
    err = err + t1 * t1;
  }
  c.q[0] = q0; c.q[1] = q1; c.err = err;
  return c;
}

// encode_candidate for a block whose scale byte and effective scale are
// nonzero and whose reciprocal is finite (ok = true): the same steps and
// float32 roundings without the branches of those cases.  ok = false means
// the caller must use encode_candidate (its result is then not used).
__device__ inline Cand encode_candidate_fast(const float* x, float amax_b, float S, float m, bool& ok) {
  Cand c;
  const float d = m * S;
  const float u = amax_b / d;
  c.sc = e4m3_rne_u(u);
  const float scf = e4m3_to_f32(c.sc);
  const float eff = scf * S;
  const float inv = 1.0f / eff;
  ok = c.sc != 0u && eff != 0.0f && !__builtin_isinf(inv);
  const float mant = mant_factor(scf);
  uint32_t q0 = 0, q1 = 0;
  float err = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; i += 2) {
    const uint32_t pk = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, x[i] * inv, x[i + 1] * inv, 1.0f, 0) & 0xFFu;
    if (i < 8) q0 |= pk << (4 * i); else q1 |= pk << (4 * (i - 8));
    const f32x2 p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(pk, scf, 0);
    const float t0 = x[i] - (p[0] * mant) * S;
    const float t1 = x[i + 1] - (p[1] * mant) * S;
    err = err + t0 * t0;
    err = err + t1 * t1;
  }
  c.q[0] = q0; c.q[1] = q1; c.err = err;
  return c;
}

// One half (8 elements) of a 16-block under candidate m, without the error
// sum: the scale byte and the 8 codes packed as 4 bytes (element 2p in the
// low nibble of byte p).  The same steps as encode_candidate, so the codes are
// identical; amax_b is the whole block's.
__device__ inline uint32_t encode_half(const float* x, float amax_b, float S, float m, uint32_t& sc_out) {
  const float d = m * S;
  const float u = amax_b / d;
  const uint32_t sc = e4m3_rne_u(u);
  sc_out = sc;
  const float scf = e4m3_to_f32(sc);
  const float eff = scf * S;
  uint32_t q = 0;
  if (sc == 0u || eff == 0.0f) {
#pragma unroll
    for (int i = 0; i < 8; ++i) q |= ((__float_as_uint(x[i]) >> 31) << 3) << (4 * i);
    return q;
  }
  const float inv = 1.0f / eff;
  const bool inv_inf = __builtin_isinf(inv);
#pragma unroll
  for (int i = 0; i < 8; i += 2) {
    float y0 = x[i] * inv, y1 = x[i + 1] * inv;
    if (inv_inf) {
      if (x[i] == 0.0f) y0 = x[i];
      if (x[i + 1] == 0.0f) y1 = x[i + 1];
    }
    q |= (__builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, y0, y1, 1.0f, 0) & 0xFFu) << (4 * i);
  }
  return q;
}

}  // namespace moe4
