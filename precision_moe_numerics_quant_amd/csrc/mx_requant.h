// MXFP8 pieces shared by the transposed requantisation kernels (device code
// only): the MX scale exponent, the exact NVFP4 dequant of one code word, and
// the stochastic-rounding quantisation of one lane's 8 columns x 32 rows.
#pragma once
#include "moe4_internal.h"

namespace moe4 {

// MX scale exponent of a block amax: least e with amax <= 448 * 2**e, clamped
// to [-127, 127]; -127 for amax = 0.
__device__ inline int mx_exponent(float amax) {
  uint32_t b = __float_as_uint(amax);
  int ex = (int)((b >> 23) & 0xFFu);
  if (ex < 9) return -127;  // amax < 2**-118 <= 448 * 2**-127
  int E = ex - 127;
  int e = ((b & 0x7FFFFFu) <= 0x600000u) ? E - 8 : E - 7;  // mantissa <= 1.75
  return e > 127 ? 127 : (e < -127 ? -127 : e);
}

// Workgroup: 4 waves over 4 consecutive MX blocks (128 padded rows) x 512
// columns.  Lane l of wave w takes columns c0 + 8l .. c0 + 8l + 7 of block w:
// one 32-bit code word (8 E2M1 codes) and one E4M3 scale byte per row, so the
// block amax of each column needs no cross-lane reduction.  The MXFP8 bytes
// are staged in LDS as [column][128 rows] (16-byte chunks XOR-swizzled by
// column) and leave as 128-byte column runs, 8 lanes per run.
namespace rq {
constexpr int WAVES = 4, THREADS = 64 * WAVES, LCOLS = 8, COLS = 64 * LCOLS, ROWS = 32 * WAVES;
__device__ inline int swz(int col, int chunk) { return chunk ^ ((col >> 3) & 7); }
}  // namespace rq

// Exact q * sc of the 8 codes of one row (byte p of cw -> columns 2p, 2p+1);
// a zero scale gives signed zeros.
__device__ inline void dequant8(uint32_t cw, uint32_t sbyte, float (&q)[8]) {
  const float scf = e4m3_to_f32(sbyte);
  const float m = scf == 0.0f ? 0.0f : mant_factor(scf);
  f32x2 d0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, scf, 0);
  f32x2 d1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, scf, 1);
  f32x2 d2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, scf, 2);
  f32x2 d3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, scf, 3);
  q[0] = d0[0] * m; q[1] = d0[1] * m; q[2] = d1[0] * m; q[3] = d1[1] * m;
  q[4] = d2[0] * m; q[5] = d2[1] * m; q[6] = d3[0] * m; q[7] = d3[1] * m;
}

// Exact values of 8 E4M3 codes of one row (byte p of w -> column p) under
// the row's E8M0 scale byte e: code * 2**(e - 127), exact in float32 (the
// smallest, 2**-9 * 2**-127, is a float32 subnormal; denormals are kept).
__device__ inline void dequant8_mx(u32x2 w, uint32_t e, float (&q)[8]) {
  const int sh = (int)e - 127;
#pragma unroll
  for (int p = 0; p < 8; ++p)
    q[p] = __builtin_amdgcn_ldexpf(e4m3_to_f32((w[p >> 2] >> (8 * (p & 3))) & 0xFFu), sh);
}

// SR E4M3 of v into byte sel of old (sel is a constant after unrolling).
__device__ inline uint32_t sr_fp8_into(uint32_t old, float v, uint32_t r, int sel) {
  switch (sel) {
    case 0: return __builtin_amdgcn_cvt_scalef32_sr_fp8_f32(old, v, r, 1.0f, 0);
    case 1: return __builtin_amdgcn_cvt_scalef32_sr_fp8_f32(old, v, r, 1.0f, 1);
    case 2: return __builtin_amdgcn_cvt_scalef32_sr_fp8_f32(old, v, r, 1.0f, 2);
    default: return __builtin_amdgcn_cvt_scalef32_sr_fp8_f32(old, v, r, 1.0f, 3);
  }
}

// Whether fl(fl(q * S) * 2^-ex) == fl(q * (S * 2^-ex)) for every dequantised
// NVFP4 value q of a block and its MX exponent ex: for 2^-100 <= S < 2^8 the
// products q * S (|q| in [2^-10, 2688] or 0) and S * 2^-ex (ex in [-118, 12]
// for a nonzero column) stay normal and finite and the result is above 2^-14,
// so scaling by the power of two commutes with rounding; a column with
// ex = -127 is then all zeros, and a factor 0 keeps the signed zeros.
__device__ inline bool fold_scale_ok(float S) { return S >= 0x1p-100f && S < 0x1p8f; }

// SR quantisation of one lane's 8 columns x nvalid rows; each group of 4
// rows leaves as one dword per column (byte i % 4 = row i) through
// put(k, column, dword), k = row group.  Rows past nvalid are zero codes.
// FAST: every element pair index of the block is below 2**32, so the
// per-pair key is the constant key0 and the index arithmetic is 32-bit (and
// j0, jstride are multiples of 4: a lane's 8 columns start at a multiple of 8
// and the row length is a multiple of 32, so Fmix32x4 applies).
// FULL: all 32 rows are valid (no row masks).
// deq(i, q) gives row i's 8 exact source values (before the factor S).
template <bool FAST, bool FULL, typename Deq, typename Put>
__device__ inline void requant_block(Deq deq, int nvalid, float S, const float (&pc)[8], int64_t j0, int64_t jstride,
                                     uint32_t base, uint32_t key0, Put put) {
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    uint32_t od[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) od[q] = 0u;
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int i = 4 * k + ii;
      if (FULL || i < nvalid) {
        float q[8];
        deq(i, q);
        const Fmix32x4 hw((uint32_t)j0 + (uint32_t)i * (uint32_t)jstride, key0);  // (used when FAST)
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          uint32_t word;
          if (FAST) {
            word = hw.word(p);
          } else {
            const int64_t j = j0 + (int64_t)i * jstride + p;
            word = fmix32((uint32_t)j ^ fmix32(base ^ (uint32_t)((uint64_t)j >> 32)));
          }
          const float v0 = q[2 * p] * S, v1 = q[2 * p + 1] * S;  // fl(fl(q*sc)*S)
          od[2 * p] = sr_fp8_into(od[2 * p], v0 * pc[2 * p], word << 16, ii);
          od[2 * p + 1] = sr_fp8_into(od[2 * p + 1], v1 * pc[2 * p + 1], word & 0xFFFF0000u, ii);
        }
      }
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) put(k, q, od[q]);
  }
}

// Store a workgroup's staged tile: lq [column][128 rows] (16-byte chunks
// swizzled by column) leaves as each column's 128-byte runs of the 4 blocks;
// lsf [column][block] as scale bytes, row-major (column stride P/32) or, with
// sfb, block-major (consecutive columns are consecutive bytes).  lblk[b] =
// {code offset at column 0, P (0: no block), scale offset at column 0}.
__device__ inline void rq_store_tile(const uint8_t* lq, const uint8_t* lsf, const int64_t (&lblk)[rq::WAVES][3],
                                     int64_t c0, int64_t C, int sfb, uint8_t* __restrict__ out_c,
                                     uint8_t* __restrict__ out_s) {
  using namespace rq;
  const int tid = threadIdx.x;
#pragma unroll 4
  for (int it = 0; it < COLS * 8 / THREADS; ++it) {
    const int idx = it * THREADS + tid;
    const int col = idx >> 3, chunk = idx & 7, b = chunk >> 1;
    const int64_t Pb = lblk[b][1], gc = c0 + col;
    if (Pb != 0 && gc < C)
      *reinterpret_cast<u32x4*>(out_c + lblk[b][0] + gc * Pb + (chunk & 1) * 16) =
          *reinterpret_cast<const u32x4*>(lq + col * ROWS + swz(col, chunk) * 16);
  }
#pragma unroll
  for (int it = 0; it < COLS * WAVES / THREADS; ++it) {
    const int idx = it * THREADS + tid;
    const int col = sfb ? idx % COLS : idx >> 2, b = sfb ? idx / COLS : idx & 3;
    const int64_t Pb = lblk[b][1], gc = c0 + col;
    if (Pb != 0 && gc < C) out_s[lblk[b][2] + (sfb ? gc : gc * (Pb / 32))] = lsf[col * WAVES + b];
  }
}

}  // namespace moe4
