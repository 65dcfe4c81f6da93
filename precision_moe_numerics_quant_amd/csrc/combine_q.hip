// Combine-path quantiser (gfx950).  The expert results travelling back for
// the combine are sent as 8-bit fixed-point values with one E8M0 scale per
// 32, 8.25 bits per value, after a Hadamard transform that spreads extreme
// values over the block (lhc.media page, paragraph on communication).
//
// Readings of the format the page names "S2F6": an int8 code c worth
// c * 2^-6, c in [-127, 127]; per 32-value block the scale exponent
// e = floor(log2 amax), clamped to [-127, 127], -127 for an all-zero block,
// stored as e + 127; codes rne(y * 2^(6 - e)) clamped to +-127.  The transform
// is the unnormalised Sylvester H_32 over the same blocks, computed in float32
// as five butterfly stages (a, b) -> (a + b, a - b) with partner distance
// 1, 2, 4, 8, 16 in that order (its rounding decides the codes).
//
// Layout of the quantiser and the decode: four lanes per block, each holding
// eight consecutive values (two 16-byte loads; a wave reads 2 KB contiguously).  Stages 1, 2, 4 stay inside
// the lane; stages 8 and 16 exchange with the lanes at xor 1 and xor 2 of the
// quad through DPP quad permutations, and so does the block maximum.  A quad
// is always wholly inside or outside the grid, so its four lanes are active
// together.  The combine instead gives each lane a whole block of one routed
// row (32 code bytes), so its k inverse transforms need no exchanges.
//
// The receiver's inverse is exact: the codes go through integer butterflies
// (every partial sum below 2^12 in magnitude) and one power-of-two scale,
// 2^(e - 6 - 5), so a decoded row is the same float32 in any order, and the
// gated sum in slot order matches the plain combine bit for bit.
#include "moe4_internal.h"

namespace moe4 {
namespace hq {
constexpr int BLOCK = 32;
constexpr int MAXK = 16;
constexpr int THREADS = 256;
}  // namespace hq

// This file's device-side error word (moe4_debug_check reads and clears it).
static __device__ uint32_t g_dev_err;
uint32_t take_dev_err_combine_q() { return take_device_word(&g_dev_err); }

// quad_perm [1,0,3,2] and [2,3,0,1]: the value of lane q ^ 1 and of lane q ^ 2
__device__ inline int quad_xor1(int v) { return __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false); }
__device__ inline int quad_xor2(int v) { return __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false); }
__device__ inline float quad_xor1(float v) { return __int_as_float(quad_xor1(__float_as_int(v))); }
__device__ inline float quad_xor2(float v) { return __int_as_float(quad_xor2(__float_as_int(v))); }

// One 32-value block's Walsh-Hadamard transform, lane q holding values
// 8q .. 8q + 7.  T is float (the sender, rounded stage by stage) or int (the
// receiver, exact).
template <typename T>
__device__ inline void fwht32_quad(T (&v)[8], int q) {
#pragma unroll
  for (int h = 1; h < 8; h <<= 1)
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (!(i & h)) {
        const T a = v[i], b = v[i + h];
        v[i] = a + b;
        v[i + h] = a - b;
      }
  // distance 8: the partner is lane q ^ 1; the lower lane keeps a + b, the
  // upper one a - b with a the lower lane's value
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const T o = quad_xor1(v[i]);
    v[i] = (q & 1) ? o - v[i] : v[i] + o;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const T o = quad_xor2(v[i]);
    v[i] = (q & 2) ? o - v[i] : v[i] + o;
  }
}

__global__ void __launch_bounds__(hq::THREADS) k_hmx8_quant(const float* __restrict__ x, int64_t n_blk,
                                                           int8_t* __restrict__ codes, uint8_t* __restrict__ sf) {
  const int64_t gid = (int64_t)blockIdx.x * hq::THREADS + threadIdx.x;
  const int64_t blk = gid >> 2;
  const int q = (int)(gid & 3);
  if (blk >= n_blk) return;
  const f32x4* p = reinterpret_cast<const f32x4*>(x + blk * hq::BLOCK + q * 8);
  const f32x4 lo = p[0], hi = p[1];
  float v[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  fwht32_quad(v, q);
  float am = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) am = fmaxf(am, fabsf(v[i]));
  am = fmaxf(am, quad_xor1(am));
  am = fmaxf(am, quad_xor2(am));
  int e = -127;
  if (am > 0.0f) {
    e = __builtin_amdgcn_frexp_expf(am) - 1;  // am = m 2^(e+1), m in [0.5, 1)
    e = e < -127 ? -127 : e;                 // (a float32 amax is below 2^128)
  }
  uint32_t w[2] = {0u, 0u};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    // |v| <= am < 2^(e+1): the scaled value is exact and below 128
    float r = __builtin_rintf(__builtin_amdgcn_ldexpf(v[i], 6 - e));
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    w[i >> 2] |= ((uint32_t)(int)r & 0xFFu) << (8 * (i & 3));
  }
  *reinterpret_cast<u32x2*>(codes + blk * hq::BLOCK + q * 8) = u32x2{w[0], w[1]};
  if (q == 0) sf[blk] = (uint8_t)(e + 127);
}

// Exact decode of lane q's eight values of one block: H_32 c * 2^(e - 11).
__device__ inline void decode_quad(u32x2 cw, uint32_t sbyte, int q, float (&out)[8]) {
  int c[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) c[i] = (int)(int8_t)(uint8_t)(cw[i >> 2] >> (8 * (i & 3)));
  fwht32_quad(c, q);
  const int sh = (int)sbyte - 127 - 6 - 5;
#pragma unroll
  for (int i = 0; i < 8; ++i) out[i] = __builtin_amdgcn_ldexpf((float)c[i], sh);
}

__global__ void __launch_bounds__(hq::THREADS) k_hmx8_dequant(const int8_t* __restrict__ codes,
                                                             const uint8_t* __restrict__ sf, int64_t n_blk,
                                                             float* __restrict__ out) {
  const int64_t gid = (int64_t)blockIdx.x * hq::THREADS + threadIdx.x;
  const int64_t blk = gid >> 2;
  const int q = (int)(gid & 3);
  if (blk >= n_blk) return;
  float v[8];
  decode_quad(*reinterpret_cast<const u32x2*>(codes + blk * hq::BLOCK + q * 8), sf[blk], q, v);
  f32x4* o = reinterpret_cast<f32x4*>(out + blk * hq::BLOCK + q * 8);
  o[0] = f32x4{v[0], v[1], v[2], v[3]};
  o[1] = f32x4{v[4], v[5], v[6], v[7]};
}

// y[t] = bf16(acc), acc = 0; for j = 0 .. k-1: acc = fl(acc + fl(g[t,j] * Yhat[row])),
// Yhat the exact decode of the payload row inv[t*k + j].  One lane per
// (token, 32-column block): the whole inverse transform stays in the lane as
// integer butterflies (no cross-lane traffic), one address product per slot,
// and the next slot's 32 code bytes are in flight while the current one is
// decoded.  Yhat = c * 2^sh exactly, so when g * 2^sh is itself exact (a
// round trip checks it) fl(g * Yhat) = fl((g * 2^sh) * c): one multiply per
// value; otherwise the value is scaled first.
__device__ inline void load_slot(const int8_t* __restrict__ codes, const uint8_t* __restrict__ sf,
                                 const float* __restrict__ gates, const int32_t* __restrict__ inv, int64_t tk,
                                 int64_t n_rows, int64_t d, int64_t b, u32x4 (&w)[2], uint32_t& s, float& g) {
  int64_t row = inv[tk];
  if (row < 0 || row >= n_rows) {
    atomicOr(&g_dev_err, MOE4_DEVERR_INDEX);
    row = row < 0 ? 0 : n_rows - 1;
  }
  g = gates[tk];
  const int64_t off = row * d + b * hq::BLOCK;
  const u32x4* p = reinterpret_cast<const u32x4*>(codes + off);
  w[0] = p[0];
  w[1] = p[1];
  s = sf[off / hq::BLOCK];
}

__global__ void __launch_bounds__(hq::THREADS) k_combine_hmx8(const int8_t* __restrict__ codes,
                                                             const uint8_t* __restrict__ sf,
                                                             const float* __restrict__ gates,
                                                             const int32_t* __restrict__ inv, int64_t T, int k,
                                                             int64_t d, int64_t n_rows, uint16_t* __restrict__ y) {
  const int64_t nb = d / hq::BLOCK;
  const int64_t gid = (int64_t)blockIdx.x * hq::THREADS + threadIdx.x;
  if (gid >= T * nb) return;
  const int64_t t = gid / nb, b = gid - t * nb;
  float acc[hq::BLOCK];
#pragma unroll
  for (int i = 0; i < hq::BLOCK; ++i) acc[i] = 0.0f;
  u32x4 w[2][2];
  uint32_t s[2];
  float g[2];
  load_slot(codes, sf, gates, inv, t * k, n_rows, d, b, w[0], s[0], g[0]);
#pragma unroll
  for (int j = 0; j < hq::MAXK; ++j) {
    if (j < k) {
      if (j + 1 < k)
        load_slot(codes, sf, gates, inv, t * k + j + 1, n_rows, d, b, w[(j + 1) & 1], s[(j + 1) & 1],
                  g[(j + 1) & 1]);
      int c[hq::BLOCK];
#pragma unroll
      for (int i = 0; i < hq::BLOCK; ++i)
        c[i] = (int)(int8_t)(uint8_t)(w[j & 1][i >> 4][(i >> 2) & 3] >> (8 * (i & 3)));
#pragma unroll
      for (int h = 1; h < hq::BLOCK; h <<= 1)
#pragma unroll
        for (int i = 0; i < hq::BLOCK; ++i)
          if (!(i & h)) {
            const int a0 = c[i], b0 = c[i + h];
            c[i] = a0 + b0;
            c[i + h] = a0 - b0;
          }
      const int sh = (int)s[j & 1] - 127 - 6 - 5;
      const float gj = g[j & 1];
      const float gs = __builtin_amdgcn_ldexpf(gj, sh);
      if (__builtin_amdgcn_ldexpf(gs, -sh) == gj) {
#pragma unroll
        for (int i = 0; i < hq::BLOCK; ++i) acc[i] = acc[i] + gs * (float)c[i];
      } else {
#pragma unroll
        for (int i = 0; i < hq::BLOCK; ++i) acc[i] = acc[i] + gj * __builtin_amdgcn_ldexpf((float)c[i], sh);
      }
    }
  }
  u32x4* o = reinterpret_cast<u32x4*>(y + t * d + b * hq::BLOCK);
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    u32x4 out;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      out[i] = f32_to_bf16_bits(acc[8 * v + 2 * i]) | (f32_to_bf16_bits(acc[8 * v + 2 * i + 1]) << 16);
    o[v] = out;
  }
}

static inline bool aligned8(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 7u) == 0; }

static unsigned quad_grid(int64_t n_quads) {
  return (unsigned)((n_quads * 4 + hq::THREADS - 1) / hq::THREADS);
}

}  // namespace moe4

using namespace moe4;

extern "C" int moe_hmx8_quant(const float* x, int64_t rows, int64_t cols, int8_t* codes, uint8_t* sf,
                              void* stream) {
  MOE4_REQUIRE(rows >= 0 && cols > 0 && cols % hq::BLOCK == 0, MOE4_EINVAL,
               "moe_hmx8_quant: bad sizes (rows >= 0, cols % 32 == 0)");
  MOE4_REQUIRE(rows == 0 || (x && codes && sf), MOE4_EINVAL, "moe_hmx8_quant: NULL pointer");
  MOE4_REQUIRE(aligned16(x) && aligned8(codes), MOE4_EALIGN,
               "moe_hmx8_quant: x must be 16-byte and codes 8-byte aligned");
  if (rows == 0) return MOE4_OK;
  const int64_t n_blk = rows * (cols / hq::BLOCK);
  MOE4_REQUIRE(n_blk * 4 / hq::THREADS < (int64_t)1 << 31, MOE4_EINVAL,
               "moe_hmx8_quant: too large");
  hipLaunchKernelGGL(k_hmx8_quant, dim3(quad_grid(n_blk)), dim3(hq::THREADS), 0, as_stream(stream), x, n_blk,
                     codes, sf);
  return check_launch("moe_hmx8_quant");
}

extern "C" int moe_hmx8_dequant(const int8_t* codes, const uint8_t* sf, int64_t rows, int64_t cols, float* out,
                                void* stream) {
  MOE4_REQUIRE(rows >= 0 && cols > 0 && cols % hq::BLOCK == 0, MOE4_EINVAL,
               "moe_hmx8_dequant: bad sizes (rows >= 0, cols % 32 == 0)");
  MOE4_REQUIRE(rows == 0 || (codes && sf && out), MOE4_EINVAL, "moe_hmx8_dequant: NULL pointer");
  MOE4_REQUIRE(aligned8(codes) && aligned16(out), MOE4_EALIGN,
               "moe_hmx8_dequant: codes must be 8-byte and out 16-byte aligned");
  if (rows == 0) return MOE4_OK;
  const int64_t n_blk = rows * (cols / hq::BLOCK);
  MOE4_REQUIRE(n_blk * 4 / hq::THREADS < (int64_t)1 << 31, MOE4_EINVAL, "moe_hmx8_dequant: too large");
  hipLaunchKernelGGL(k_hmx8_dequant, dim3(quad_grid(n_blk)), dim3(hq::THREADS), 0, as_stream(stream), codes, sf,
                     n_blk, out);
  return check_launch("moe_hmx8_dequant");
}

extern "C" int moe_combine_hmx8(const int8_t* codes, const uint8_t* sf, const float* gates,
                                const int32_t* inv_perm, int64_t T, int32_t k, int64_t d, uint16_t* y,
                                void* stream) {
  MOE4_REQUIRE(T >= 0 && k >= 1 && k <= hq::MAXK && d > 0 && d % hq::BLOCK == 0, MOE4_EINVAL,
               "moe_combine_hmx8: bad sizes (1 <= k <= 16, d % 32 == 0)");
  MOE4_REQUIRE(T == 0 || (codes && sf && gates && inv_perm && y), MOE4_EINVAL, "moe_combine_hmx8: NULL pointer");
  MOE4_REQUIRE(aligned16(codes) && aligned16(y), MOE4_EALIGN,
               "moe_combine_hmx8: codes and y must be 16-byte aligned");
  if (T == 0) return MOE4_OK;
  const int64_t n_blk = T * (d / hq::BLOCK);
  MOE4_REQUIRE(n_blk / hq::THREADS < (int64_t)1 << 31, MOE4_EINVAL, "moe_combine_hmx8: too large");
  hipLaunchKernelGGL(k_combine_hmx8, dim3((unsigned)((n_blk + hq::THREADS - 1) / hq::THREADS)), dim3(hq::THREADS), 0,
                     as_stream(stream), codes, sf, gates, inv_perm, T, k, d, T * (int64_t)k, y);
  return check_launch("moe_combine_hmx8");
}
