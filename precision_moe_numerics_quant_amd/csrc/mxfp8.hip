// MXFP8 quantisation kernels (gfx950): the transposed stochastic-rounding
// requantisation of NVFP4 forward operands, and the row-wise / transposed
// quantisation of gradients.
//
// The requantisation follows the lhc.media page's description of the backward
// pass (dequantise the forward values, transpose them at higher precision,
// requantise into MXFP8 with stochastic rounding, because the transpose
// regroups the values that share a scale).  MXFP8 = E4M3 elements with one E8M0
// scale per 32 values, the 32 running along the GEMM contraction, which after
// the transpose is the token (row) dimension of each expert group.
//
// Tiling of the transposed kernels: a workgroup of 256 threads takes 32
// padded rows (one MX block, never straddling a group) x 128 columns.  The
// tile is staged through LDS transposed; each wave then owns 32 columns, each
// lane an adjacent column pair over 8 rows, so the pair shares one 32-bit
// random word and the lane writes 8 contiguous output bytes per column.  The
// block amax is a 4-lane reduction (xor 16, xor 32).
#include "act.h"
#include "gemm_common.h"
#include "moe4_internal.h"
#include "mx_requant.h"

namespace moe4 {

constexpr int TR = 32;    // rows per tile (one MX block)
constexpr int TC = 128;   // columns per tile
constexpr int MXT = 256;  // threads
constexpr int MX_T_CPW = 4;  // column tiles per workgroup of the transposed kernels that stage a table

__device__ inline int find_group(const int32_t* off, int G, int64_t r) {
  int lo = 0, hi = G - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if ((int64_t)off[mid] <= r) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// E4M3 byte of w (|w| <= 448): RNE, or SR with the 16-bit word r16.
template <bool SR>
__device__ inline uint32_t mx_round(float w, uint32_t r16) {
  if (SR)
    return (uint32_t)__builtin_amdgcn_cvt_scalef32_sr_fp8_f32(0, w, r16 << 16, 1.0f, 0) & 0xFFu;
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(w, 0.0f, 0, false) & 0xFFu;
}

// Four consecutive values, already scaled, as one word of E4M3 bytes (value i
// in byte i): RNE two values per conversion, SR each into its byte, with the
// pair words' halves as random bits as in mx_round (w0: values 0, 1; w1: 2, 3).
template <bool SR>
__device__ inline uint32_t mx_word4(float a, float b, float c, float d, uint32_t w0, uint32_t w1) {
  if (SR) {
    uint32_t o = __builtin_amdgcn_cvt_scalef32_sr_fp8_f32(0, a, w0 << 16, 1.0f, 0);
    o = __builtin_amdgcn_cvt_scalef32_sr_fp8_f32(o, b, w0 & 0xFFFF0000u, 1.0f, 1);
    o = __builtin_amdgcn_cvt_scalef32_sr_fp8_f32(o, c, w1 << 16, 1.0f, 2);
    return __builtin_amdgcn_cvt_scalef32_sr_fp8_f32(o, d, w1 & 0xFFFF0000u, 1.0f, 3);
  }
  const uint32_t o = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, (int)o, true);
}

// Random word of element pair j = i >> 1 (base = seed/stream key).
__device__ inline uint32_t sr_word(uint32_t base, uint64_t j) {
  uint32_t key = fmix32(base ^ (uint32_t)(j >> 32));
  return fmix32((uint32_t)j ^ key);
}

// Quantise, for one lane, 8 rows x 2 adjacent columns (c, c+1) of values
// v[row][0..1] that belong to one 32-row MX block shared with the lanes at
// xor 16 and xor 32; writes 8 code bytes per column and (rseg == 0) the
// scale bytes.  src_row0: source row of the lane's first row (only for SR
// indices); rows beyond the group are zeros already.
template <bool SR>
__device__ inline void mx_quant_pair_T(const float (&v)[8][2], int rseg, int64_t src_row0, int64_t C, int64_t c,
                                       uint32_t base, uint8_t* out_c0, uint8_t* out_c1, uint8_t* sf_c0,
                                       uint8_t* sf_c1) {
  float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a0 = fmaxf(a0, fabsf(v[i][0]));
    a1 = fmaxf(a1, fabsf(v[i][1]));
  }
  a0 = max_xor32(max_xor16(a0));
  a1 = max_xor32(max_xor16(a1));
  const int e0 = mx_exponent(a0), e1 = mx_exponent(a1);
  const float p0 = __builtin_amdgcn_ldexpf(1.0f, -e0), p1 = __builtin_amdgcn_ldexpf(1.0f, -e1);
  uint32_t lo0 = 0, hi0 = 0, lo1 = 0, hi1 = 0;
  if (SR) {
    // pair index of (row src_row0 + i, column c): j0 + i C / 2 (c even)
    const uint64_t j0 = (uint64_t)(src_row0 * C + c) >> 1;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t word = sr_word(base, j0 + (uint64_t)i * (uint64_t)(C >> 1));
      const uint32_t b0 = mx_round<SR>(v[i][0] * p0, word & 0xFFFFu);
      const uint32_t b1 = mx_round<SR>(v[i][1] * p1, word >> 16);
      if (i < 4) { lo0 |= b0 << (8 * i); lo1 |= b1 << (8 * i); }
      else { hi0 |= b0 << (8 * (i - 4)); hi1 |= b1 << (8 * (i - 4)); }
    }
  } else {  // RNE, two values per conversion (each value converted on its own)
    lo0 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v[0][0] * p0, v[1][0] * p0, 0, false);
    lo0 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v[2][0] * p0, v[3][0] * p0, (int)lo0, true);
    hi0 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v[4][0] * p0, v[5][0] * p0, 0, false);
    hi0 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v[6][0] * p0, v[7][0] * p0, (int)hi0, true);
    lo1 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v[0][1] * p1, v[1][1] * p1, 0, false);
    lo1 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v[2][1] * p1, v[3][1] * p1, (int)lo1, true);
    hi1 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v[4][1] * p1, v[5][1] * p1, 0, false);
    hi1 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v[6][1] * p1, v[7][1] * p1, (int)hi1, true);
  }
  *reinterpret_cast<u32x2*>(out_c0) = u32x2{lo0, hi0};
  *reinterpret_cast<u32x2*>(out_c1) = u32x2{lo1, hi1};
  if (rseg == 0) {
    *sf_c0 = (uint8_t)(e0 + 127);
    *sf_c1 = (uint8_t)(e1 + 127);
  }
}

// Tile coordinates shared by the transposed kernels.  Returns false if the
// tile lies beyond the padded extent.
struct TileT {
  int g;
  int64_t pr_in_g;   // first padded row of the tile within its group
  int64_t P;         // padded rows of the group
  int64_t src0;      // source row of the tile's first row
  int64_t nvalid;    // valid (unpadded) rows in the tile (0..32)
  int64_t out_base;  // code offset of the group block
};

// A padded extent beyond max_pr (the caller's output size) or a group end past
// R source rows violates the call's preconditions: such tiles are skipped or
// clamped, never accessed out of bounds.
__device__ inline bool tile_coords(const int32_t* off, const int32_t* offp, int G, int64_t C, int64_t R,
                                   int64_t max_pr, int64_t rt, TileT& t) {
  const int64_t pr = rt * TR;
  if (pr >= (int64_t)offp[G] || (int64_t)offp[G] > max_pr) return false;
  t.g = find_group(offp, G, pr);
  t.pr_in_g = pr - offp[t.g];
  t.P = (int64_t)offp[t.g + 1] - offp[t.g];
  t.src0 = (int64_t)off[t.g] + t.pr_in_g;
  const int64_t gend = (int64_t)off[t.g + 1] < R ? (int64_t)off[t.g + 1] : R;
  int64_t n = gend - t.src0;
  t.nvalid = n < 0 ? 0 : (n > TR ? TR : n);
  t.out_base = C * (int64_t)offp[t.g];
  return true;
}

// ---------------------------------------------------------------- requant-T
// MX: the source is MXFP8 row-wise (codes [R, C], E8M0 scales [R, C/32], no
// tensor scale: S = 1) instead of NVFP4.
template <bool MX>
__global__ void __launch_bounds__(rq::THREADS) k_requant_T(const uint8_t* __restrict__ codes,
                                                           const uint8_t* __restrict__ sf,
                                                           const float* __restrict__ ts, int ts_per_group, int64_t C,
                                                           const int32_t* __restrict__ off,
                                                           const int32_t* __restrict__ offp, int G, int64_t R,
                                                           int64_t max_pr, int64_t n_ct, uint32_t base, int sfb,
                                                           uint8_t* __restrict__ out_c, uint8_t* __restrict__ out_s) {
  using namespace rq;
  __shared__ __attribute__((aligned(16))) uint8_t lq[COLS * ROWS];
  __shared__ uint8_t lsf[COLS * WAVES];  // [column][block]
  __shared__ int64_t lblk[WAVES][3];     // block's code offset at column 0, P (0: no block), scale offset at column 0
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int64_t c0 = (int64_t)(blockIdx.x % n_ct) * COLS;
  const int64_t pr = ((int64_t)(blockIdx.x / n_ct) * WAVES + w) * 32;
  const int64_t ptot = offp[G];
  const bool present = pr < ptot && ptot <= max_pr;
  int64_t P = 0, pr_in_g = 0, src0 = 0, obase = 0, sbase = 0;
  int nvalid = 0, g = 0;
  if (present) {
    g = find_group(offp, G, pr);
    pr_in_g = pr - offp[g];
    P = (int64_t)offp[g + 1] - offp[g];
    src0 = (int64_t)off[g] + pr_in_g;
    const int64_t gend = (int64_t)off[g + 1] < R ? (int64_t)off[g + 1] : R;
    const int64_t n = gend - src0;
    nvalid = n < 0 ? 0 : (n > 32 ? 32 : (int)n);
    obase = C * (int64_t)offp[g] + pr_in_g;
    sbase = C * (int64_t)offp[g] / 32 + (sfb ? (pr_in_g / 32) * C : pr_in_g / 32);
  }
  if (l == 0) {
    lblk[w][0] = obase;
    lblk[w][1] = P;
    lblk[w][2] = sbase;
  }
  const int64_t c = c0 + LCOLS * l;
  // row group k (rows 4k..4k+3 of block w) of column col: dword k % 4 of
  // 16-byte chunk 2w + k / 4 of the column's LDS run
  auto put = [&](int k, int q, uint32_t v) {
    const int col = LCOLS * l + q;
    *reinterpret_cast<uint32_t*>(lq + col * ROWS + swz(col, 2 * w + (k >> 2)) * 16 + (k & 3) * 4) = v;
  };
  int ex[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) ex[q] = -127;
  if (nvalid > 0 && c < C) {
    // code words (NVFP4: 8 E2M1 codes in one dword; MXFP8: 8 E4M3 bytes in
    // two); scale bytes packed 4 rows per register
    uint32_t cw[32][MX ? 2 : 1], sbp[8];
    const uint8_t* crow = MX ? codes + src0 * C + c : codes + src0 * (C / 2) + c / 2;
    const uint8_t* srow = MX ? sf + src0 * (C / 32) + c / 32 : sf + src0 * (C / 16) + c / 16;
#pragma unroll
    for (int k = 0; k < 8; ++k) sbp[k] = 0u;
#pragma unroll
    for (int i = 0; i < 32; ++i) {  // rows past the group repeat its last row and are never used
      const int64_t ri = i < nvalid ? i : nvalid - 1;
      if (MX) {
        const u32x2 wv = *reinterpret_cast<const u32x2*>(crow + ri * C);
        cw[i][0] = wv[0];
        cw[i][MX ? 1 : 0] = wv[1];
      } else {
        cw[i][0] = *reinterpret_cast<const uint32_t*>(crow + ri * (C / 2));
      }
      sbp[i >> 2] |= (uint32_t)srow[ri * (MX ? C / 32 : C / 16)] << (8 * (i & 3));
    }
    const float S = MX ? 1.0f : ts[ts_per_group ? g : 0];
    auto deq = [&](int i, float (&q)[8]) {
      const uint32_t sb = (sbp[i >> 2] >> (8 * (i & 3))) & 0xFFu;
      if (MX) dequant8_mx(u32x2{cw[i][0], cw[i][MX ? 1 : 0]}, sb, q);
      else dequant8(cw[i][0], sb, q);
    };
    // block amax of fl(fl(q*sc)*S) per column: fl(max |q*sc| * S), as
    // rounding a product by S > 0 keeps the order of the exact q*sc
    float am[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) am[q] = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      if (i < nvalid) {
        float q8[8];
        deq(i, q8);
#pragma unroll
        for (int q = 0; q < 8; ++q) am[q] = fmaxf(am[q], fabsf(q8[q]));
      }
    }
    float pc[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      ex[q] = mx_exponent(am[q] * S);
      pc[q] = __builtin_amdgcn_ldexpf(1.0f, -ex[q]);
    }
    if (MX) {  // decode again below instead of keeping the 256 decoded values live
#pragma unroll
      for (int i = 0; i < 32; ++i) asm volatile("" : "+v"(cw[i][0]), "+v"(cw[i][MX ? 1 : 0]));
    }
    const int64_t j0 = src0 * (C / 2) + c / 2;  // pair index of (row src0, column c)
    const uint32_t key0 = fmix32(base);
    const bool fast = j0 + 31 * (C / 2) + 3 < ((int64_t)1 << 32);
    if (!MX && fast && nvalid == 32 && fold_scale_ok(S)) {  // one multiply by S * 2^-ex per value
      float f[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) f[q] = ex[q] == -127 ? 0.0f : S * pc[q];
      requant_block<true, true>(deq, nvalid, 1.0f, f, j0, C / 2, base, key0, put);
    } else if (fast && nvalid == 32)
      requant_block<true, true>(deq, nvalid, S, pc, j0, C / 2, base, key0, put);
    else if (fast)
      requant_block<true, false>(deq, nvalid, S, pc, j0, C / 2, base, key0, put);
    else
      requant_block<false, false>(deq, nvalid, S, pc, j0, C / 2, base, key0, put);
  } else {  // no valid rows (padding block or columns past C): zero codes
#pragma unroll
    for (int k = 0; k < 8; ++k)
#pragma unroll
      for (int q = 0; q < 8; ++q) put(k, q, 0u);
  }
#pragma unroll
  for (int q = 0; q < 8; ++q) lsf[(LCOLS * l + q) * WAVES + w] = (uint8_t)(ex[q] + 127);
  __syncthreads();
  rq_store_tile(lq, lsf, lblk, c0, C, sfb, out_c, out_s);
}

// ------------------------------------------ weights of the MXFP8 forward
// Float32 weights [G * grows, C] -> the row-wise MXFP8 RNE copy (blocks of 32
// along the row, the forward contraction: the bytes of k_mx_rows) and, from
// those codes with the same steps as k_requant_T<true>, the transposed MXFP8
// SR copy (group-major, grows rows per group, row-major scales), in one read
// of the weights.  MXFP8 has no tensor scale, so no tile waits for the rest
// of its group.  Tile: 4 waves x (32 rows = one transposed MX block) x 512
// columns of one group; lane l of wave w takes columns c0 + 8l .. c0 + 8l + 7
// of the wave's 32 rows, so lanes 4m .. 4m + 3 hold one row-wise 32-block
// (its amax through two shuffles) and each lane keeps its 32 rows' code bytes
// for the transposed requantisation.
__global__ void __launch_bounds__(rq::THREADS) __attribute__((amdgpu_waves_per_eu(2, 2)))
k_mx_quant_requant_T(const float* __restrict__ x, int64_t C, int64_t grows, uint32_t n_ct, uint32_t n_rt,
                     uint32_t base, uint8_t* __restrict__ codes, uint8_t* __restrict__ sf,
                     uint8_t* __restrict__ out_c, uint8_t* __restrict__ out_s) {
  using namespace rq;
  __shared__ __attribute__((aligned(16))) uint8_t lq[COLS * ROWS];
  __shared__ uint8_t lsf[COLS * WAVES];  // [column][block]
  __shared__ int64_t lblk[WAVES][3];
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const uint32_t ct = blockIdx.x % n_ct, rest = blockIdx.x / n_ct, rt = rest % n_rt, g = rest / n_rt;
  const int64_t c0 = (int64_t)ct * COLS, pr = (int64_t)rt * ROWS + 32 * w;  // wave's first row in g
  const bool present = pr < grows;
  const int64_t r0 = (int64_t)g * grows + pr;
  if (l == 0) {
    lblk[w][0] = C * (int64_t)g * grows + pr;
    lblk[w][1] = present ? grows : 0;
    lblk[w][2] = C * (int64_t)g * grows / 32 + pr / 32;
  }
  const int64_t c = c0 + LCOLS * l;
  auto put = [&](int k, int q, uint32_t v) {
    const int col = LCOLS * l + q;
    *reinterpret_cast<uint32_t*>(lq + col * ROWS + swz(col, 2 * w + (k >> 2)) * 16 + (k & 3) * 4) = v;
  };
  int ex[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) ex[q] = -127;
  if (present && c < C) {  // (C % 32 == 0: the four lanes of a row block agree)
    const float* xr = x + r0 * C + c;
    u32x2 cw[32];
    uint32_t sbp[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) sbp[k] = 0u;
    f32x4 vb[2][4][2];
    auto load_group = [&](int k, f32x4 (&b)[4][2]) {
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const f32x4* p = reinterpret_cast<const f32x4*>(xr + (int64_t)(4 * k + ii) * C);
        b[ii][0] = p[0];
        b[ii][1] = p[1];
      }
    };
    load_group(0, vb[0]);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if (k + 1 < 8) load_group(k + 1, vb[(k + 1) & 1]);
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int i = 4 * k + ii;
        float v[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[e] = vb[k & 1][ii][0][e];
          v[4 + e] = vb[k & 1][ii][1][e];
        }
        float a = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) a = fmaxf(a, fabsf(v[e]));
        a = fmaxf(a, lane_xor1(a));  // the row block's other three lanes
        a = fmaxf(a, lane_xor2(a));
        const int e = mx_exponent(a);
        const float p = __builtin_amdgcn_ldexpf(1.0f, -e);
        // RNE per value, two values per conversion (bytes 0-1, then 2-3)
        uint32_t lo = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v[0] * p, v[1] * p, 0, false);
        lo = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v[2] * p, v[3] * p, (int)lo, true);
        uint32_t hi = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v[4] * p, v[5] * p, 0, false);
        hi = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v[6] * p, v[7] * p, (int)hi, true);
        cw[i] = u32x2{lo, hi};
        *reinterpret_cast<u32x2*>(codes + (r0 + i) * C + c) = cw[i];
        if ((l & 3) == 0) sf[(r0 + i) * (C / 32) + c / 32] = (uint8_t)(e + 127);
        sbp[k] |= (uint32_t)(e + 127) << (8 * ii);
      }
    }
    auto deq = [&](int i, float (&q)[8]) { dequant8_mx(cw[i], (sbp[i >> 2] >> (8 * (i & 3))) & 0xFFu, q); };
    float am[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) am[q] = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      float q8[8];
      deq(i, q8);
#pragma unroll
      for (int q = 0; q < 8; ++q) am[q] = fmaxf(am[q], fabsf(q8[q]));
    }
    float pc[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      ex[q] = mx_exponent(am[q]);
      pc[q] = __builtin_amdgcn_ldexpf(1.0f, -ex[q]);
    }
    // decode again below instead of keeping the 256 decoded values live
#pragma unroll
    for (int i = 0; i < 32; ++i) asm volatile("" : "+v"(cw[i][0]), "+v"(cw[i][1]));
    const int64_t j0 = r0 * (C / 2) + c / 2;  // pair index of (row r0, column c)
    const uint32_t key0 = fmix32(base);
    if (j0 + 31 * (C / 2) + 3 < ((int64_t)1 << 32))
      requant_block<true, true>(deq, 32, 1.0f, pc, j0, C / 2, base, key0, put);
    else
      requant_block<false, true>(deq, 32, 1.0f, pc, j0, C / 2, base, key0, put);
  } else {  // rows past the group or columns past C: zero codes
#pragma unroll
    for (int k = 0; k < 8; ++k)
#pragma unroll
      for (int q = 0; q < 8; ++q) put(k, q, 0u);
  }
#pragma unroll
  for (int q = 0; q < 8; ++q) lsf[(LCOLS * l + q) * WAVES + w] = (uint8_t)(ex[q] + 127);
  __syncthreads();
  rq_store_tile(lq, lsf, lblk, c0, C, 0, out_c, out_s);
}

// ------------------------------------------------------ gradient value loads
// Source value of output row r, columns c..c+3 (float32).
struct GradSrc {
  const void* x;
  int dtype;
  const int32_t* row_map;
  int map_div;
  const float* row_scale;
  const uint16_t* dsilu_src;
};

template <int DT>
__device__ inline f32x4 load4(const void* x, int64_t idx) {
  if (DT == MOE4_F32) return *reinterpret_cast<const f32x4*>(static_cast<const float*>(x) + idx);
  u32x2 w = *reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(x) + idx);
  return f32x4{bf16_bits_to_f32(w[0] & 0xFFFFu), bf16_bits_to_f32(w[0] >> 16), bf16_bits_to_f32(w[1] & 0xFFFFu),
               bf16_bits_to_f32(w[1] >> 16)};
}

template <int DT, int MODE>  // MODE 0: plain, 1: row map + scale, 2: x * dsilu(u), 3: silu(x) (x bf16)
__device__ inline f32x4 grad_vals4(const GradSrc& g, int64_t r, int64_t C, int64_t c, const float* dtab) {
  if (MODE == 1) {
    const int32_t a = g.row_map[r];
    const float sc = g.row_scale ? g.row_scale[a] : 1.0f;
    f32x4 v = load4<DT>(g.x, (int64_t)(a / g.map_div) * C + c);
    return f32x4{sc * v[0], sc * v[1], sc * v[2], sc * v[3]};
  } else if (MODE == 2) {
    f32x4 v = load4<DT>(g.x, r * C + c);
    const u32x2 u = *reinterpret_cast<const u32x2*>(g.dsilu_src + r * C + c);
    const uint32_t uu[2] = {u[0], u[1]};
    float d[4];
    act_eval_packed<true>(uu, dtab, d);
    return f32x4{v[0] * d[0], v[1] * d[1], v[2] * d[2], v[3] * d[3]};
  } else if (MODE == 3) {  // (the table is the silu one)
    const u32x2 u = *reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(g.x) + r * C + c);
    const uint32_t uu[2] = {u[0], u[1]};
    float a[4];
    act_eval_packed<false>(uu, dtab, a);
    return f32x4{a[0], a[1], a[2], a[3]};
  }
  return load4<DT>(g.x, r * C + c);
}

// grad_vals4 for 16 consecutive columns c .. c + 15 (c % 16 == 0, C % 16 ==
// 0) in two parts, so that a tile's loads can be in flight while the previous
// tile is quantised: grad_load16 resolves the source row (and its map and
// scale) once and issues 16-byte loads, grad_finish16 makes the 16 values;
// dtab is the narrow table (stage_act_table_narrow).
struct GradRaw {
  u32x4 w[4];  // the source values (bf16: w[0..1]; float32: w[0..3])
  u32x4 u[2];  // MODE 2: the bf16 patterns of U
  float sc;    // MODE 1: the row's scale
};

template <int DT, int MODE>
__device__ inline void grad_load16(const GradSrc& g, int64_t r, int64_t C, int64_t c, GradRaw& q) {
  int64_t src = r;
  q.sc = 1.0f;
  if (MODE == 1) {
    const int32_t a = g.row_map[r];
    if (g.row_scale) q.sc = g.row_scale[a];
    src = a / g.map_div;
  }
  const int64_t idx = src * C + c;
  if (MODE == 3 || DT != MOE4_F32) {  // (bf16 bits)
    const u32x4* p = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(g.x) + idx);
    q.w[0] = p[0];
    q.w[1] = p[1];
  } else {
    const u32x4* p = reinterpret_cast<const u32x4*>(static_cast<const float*>(g.x) + idx);
#pragma unroll
    for (int k = 0; k < 4; ++k) q.w[k] = p[k];
  }
  if (MODE == 2) {
    const u32x4* pu = reinterpret_cast<const u32x4*>(g.dsilu_src + r * C + c);
    q.u[0] = pu[0];
    q.u[1] = pu[1];
  }
}

template <int DT, int MODE>
__device__ inline void grad_finish16(const GradRaw& q, const float* dtab, float (&v)[16]) {
  if (MODE == 3) {
#pragma unroll
    for (int k = 0; k < 2; ++k)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[8 * k + 2 * j] = act_eval_narrow<false>(q.w[k][j] & 0xFFFFu, dtab);
        v[8 * k + 2 * j + 1] = act_eval_narrow<false>(q.w[k][j] >> 16, dtab);
      }
    return;
  }
  if (DT == MOE4_F32) {
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int j = 0; j < 4; ++j) v[4 * k + j] = __uint_as_float(q.w[k][j]);
  } else {
#pragma unroll
    for (int k = 0; k < 2; ++k)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[8 * k + 2 * j] = bf16_bits_to_f32(q.w[k][j] & 0xFFFFu);
        v[8 * k + 2 * j + 1] = bf16_bits_to_f32(q.w[k][j] >> 16);
      }
  }
  if (MODE == 1) {
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = q.sc * v[i];
  } else if (MODE == 2) {
#pragma unroll
    for (int k = 0; k < 2; ++k)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[8 * k + 2 * j] = v[8 * k + 2 * j] * act_eval_narrow<true>(q.u[k][j] & 0xFFFFu, dtab);
        v[8 * k + 2 * j + 1] = v[8 * k + 2 * j + 1] * act_eval_narrow<true>(q.u[k][j] >> 16, dtab);
      }
  }
}

// ------------------------------------------------- row-wise gradient quant
template <int DT, int MODE, bool SR>
__global__ void __launch_bounds__(256) k_mx_rows(GradSrc g, int64_t R, int64_t C, uint32_t base,
                                                 uint8_t* __restrict__ out_c, uint8_t* __restrict__ out_s,
                                                 const float* __restrict__ act_tab) {
  __shared__ float tab[MODE >= 2 ? ACT_TAB : 1];
  if (MODE >= 2) stage_act_table(tab, act_tab);
  const int64_t nbr = C / 32;
  const int64_t blk = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (blk >= R * nbr) return;
  const int64_t r = blk / nbr, c0 = (blk % nbr) * 32;
  float v[32];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    f32x4 t = grad_vals4<DT, MODE>(g, r, C, c0 + 4 * q, tab);
    v[4 * q] = t[0]; v[4 * q + 1] = t[1]; v[4 * q + 2] = t[2]; v[4 * q + 3] = t[3];
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const int e = mx_exponent(amax);
  const float p = __builtin_amdgcn_ldexpf(1.0f, -e);
  uint32_t outw[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    uint32_t w0 = 0, w1 = 0;
    if (SR) {
      const uint64_t i0 = (uint64_t)(r * C + c0 + 4 * q);
      w0 = sr_word(base, i0 >> 1);
      w1 = sr_word(base, (i0 >> 1) + 1);
    }
    outw[q] = mx_word4<SR>(v[4 * q] * p, v[4 * q + 1] * p, v[4 * q + 2] * p, v[4 * q + 3] * p, w0, w1);
  }
  u32x4* o = reinterpret_cast<u32x4*>(out_c + r * C + c0);
  o[0] = u32x4{outw[0], outw[1], outw[2], outw[3]};
  o[1] = u32x4{outw[4], outw[5], outw[6], outw[7]};
  out_s[blk] = (uint8_t)(e + 127);
}

// ------------------------------------------------- transposed gradient quant
// ROWS: the same tile also gives the row-wise quantisation of its valid rows
// (the output of k_mx_rows for the same source, rounding and key), written to
// row_c [R, C] / row_s [R, C/32]: both operands of a gradient from one read.
// Every source row lies in one group's tile rows when off[G] == R.
template <int DT, int MODE, bool SR, bool ROWS>
__global__ void __launch_bounds__(MXT) k_mx_T(GradSrc g, int64_t R, int64_t C, const int32_t* __restrict__ off,
                                              const int32_t* __restrict__ offp, int G, int64_t max_pr, int64_t n_ct,
                                              int cpw, uint32_t base, int sfb,
                                              uint8_t* __restrict__ out_c, uint8_t* __restrict__ out_s,
                                              const float* __restrict__ act_tab, uint8_t* __restrict__ row_c,
                                              uint8_t* __restrict__ row_s) {
  __shared__ float tab[MODE >= 2 ? ACT_NARROW : 1];  // (the narrow table: LDS for four workgroups per CU)
  __shared__ float lv[TC][TR + 1];  // [column][row]
  if (MODE >= 2) stage_act_table_narrow(tab, act_tab);
  // Tile order.  Each column's output run of a 32-row tile is 32 bytes, a
  // quarter line: for sources read in place, the four row tiles of a 128-row
  // span with the same columns run back to back on one XCD (contiguous tile
  // runs per XCD), so its L2 merges the quarters into whole lines before they
  // go out.  For gathered rows (MODE 1) the column tiles of one row tile run
  // together instead, so they share the gathered source rows in L2 (measured:
  // each order is the faster one for its mode).  A workgroup takes cpw
  // column tiles of its row tile in turn (the table staged once; each tile's
  // source loads issued while the previous tile is quantised).
  const int64_t n_cw = (n_ct + cpw - 1) / cpw;
  int64_t cw, rt;
  if (MODE == 1) {
    cw = blockIdx.x % n_cw;
    rt = blockIdx.x / n_cw;
  } else {
    const int64_t n_all = (int64_t)gridDim.x / N_XCD * N_XCD;
    const int64_t b = xcd_tile(blockIdx.x, n_all), span = b / (4 * n_cw), in_span = b - span * 4 * n_cw;
    cw = in_span >> 2;
    rt = span * 4 + (in_span & 3);
  }
  TileT t;
  if (!tile_coords(off, offp, G, C, R, max_pr, rt, t)) return;
  const int tid = threadIdx.x;
  const int64_t ct0 = cw * cpw, ct_end = (cw + 1) * cpw < n_ct ? (cw + 1) * cpw : n_ct;
  // staging: thread -> row tid/8, 16 columns at (tid%8)*16 of every column tile
  const int srr = tid >> 3, scc = (tid & 7) * 16;
  auto staged = [&](int64_t ct) { return srr < t.nvalid && ct * TC + scc < C; };
  auto load = [&](int64_t ct, GradRaw& q) {
    if (staged(ct)) grad_load16<DT, MODE>(g, t.src0 + srr, C, ct * TC + scc, q);
  };
  auto tile = [&](int64_t ct, const GradRaw& q) {
    const int64_t c0 = ct * TC;
    if (ct != ct0) __syncthreads();  // (the previous tile's readers are done with lv)
    {
      const int rr = srr, cc = scc;
      float v[16];
      if (staged(ct)) {
        grad_finish16<DT, MODE>(q, tab, v);
      } else {
#pragma unroll
        for (int j = 0; j < 16; ++j) v[j] = 0.0f;
      }
#pragma unroll
      for (int j = 0; j < 16; ++j) lv[cc + j][rr] = v[j];
    }
    __syncthreads();
    if (ROWS) {  // thread pair -> (row, 32-column block); each thread 16 columns
      const int pair = tid >> 1, half = tid & 1, rr = pair >> 2, blk = pair & 3, cl0 = 32 * blk + 16 * half;
      if (rr < t.nvalid && c0 + 32 * blk < C) {  // (C % 32 == 0: whole blocks; both threads of a pair agree)
        float v[16];
        float a = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          v[i] = lv[cl0 + i][rr];
          a = fmaxf(a, fabsf(v[i]));
        }
        a = fmaxf(a, lane_xor1(a));
        const int e = mx_exponent(a);
        const float p = __builtin_amdgcn_ldexpf(1.0f, -e);
        const int64_t r_out = t.src0 + rr, cg = c0 + cl0;
        uint32_t ow[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          uint32_t w0 = 0, w1 = 0;
          if (SR) {
            const uint64_t i0 = (uint64_t)(r_out * C + cg + 4 * q);
            w0 = sr_word(base, i0 >> 1);
            w1 = sr_word(base, (i0 >> 1) + 1);
          }
          ow[q] = mx_word4<SR>(v[4 * q] * p, v[4 * q + 1] * p, v[4 * q + 2] * p, v[4 * q + 3] * p, w0, w1);
        }
        *reinterpret_cast<u32x4*>(row_c + r_out * C + cg) = u32x4{ow[0], ow[1], ow[2], ow[3]};
        if (half == 0) row_s[r_out * (C / 32) + cg / 32] = (uint8_t)(e + 127);
      }
    }
    const int w = tid >> 6, l = tid & 63;
    if (c0 + 32 * w >= C) return;
    const int cp = l & 15, rseg = l >> 4;
    const int cl = 32 * w + 2 * cp;
    float v[8][2];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      v[i][0] = lv[cl][rseg * 8 + i];
      v[i][1] = lv[cl + 1][rseg * 8 + i];
    }
    const int64_t c = c0 + cl;
    const int64_t orow = t.pr_in_g + rseg * 8;
    uint8_t* o0 = out_c + t.out_base + c * t.P + orow;
    // scale of (column c, block pr_in_g / 32): row-major [C][P/32] or block-major [P/32][C]
    uint8_t* s0 = out_s + t.out_base / 32 + (sfb ? (t.pr_in_g / 32) * C + c : c * (t.P / 32) + t.pr_in_g / 32);
    mx_quant_pair_T<SR>(v, rseg, t.src0 + rseg * 8, C, c, base, o0, o0 + t.P, s0, s0 + (sfb ? 1 : t.P / 32));
  };
  if constexpr (MODE >= 2) {
    // several column tiles per workgroup: the next tile's loads in flight
    // while a tile is staged and quantised (two named register sets, not
    // indexed by the tile's parity)
    GradRaw qa, qb;
    load(ct0, qa);
    for (int64_t ct = ct0; ct < ct_end; ct += 2) {
      if (ct + 1 < ct_end) load(ct + 1, qb);
      tile(ct, qa);
      if (ct + 1 >= ct_end) break;
      if (ct + 2 < ct_end) load(ct + 2, qa);
      tile(ct + 1, qb);
    }
  } else {  // (one tile per workgroup: a second set would only cost occupancy)
    for (int64_t ct = ct0; ct < ct_end; ++ct) {
      GradRaw q;
      load(ct, q);
      tile(ct, q);
    }
  }
}

template <int DT, int MODE>
static void launch_grad(int transpose, bool sr, const GradSrc& g, int64_t R, int64_t C, const int32_t* off,
                        const int32_t* offp, int G, int64_t max_pr, uint32_t base, uint8_t* oc, uint8_t* os,
                        const float* tab, hipStream_t s, uint8_t* rc = nullptr, uint8_t* rs = nullptr) {
  if (!transpose) {
    const int64_t nblk = R * (C / 32);
    dim3 grid((unsigned)((nblk + 255) / 256));
    if (sr) hipLaunchKernelGGL((k_mx_rows<DT, MODE, true>), grid, dim3(256), 0, s, g, R, C, base, oc, os, tab);
    else hipLaunchKernelGGL((k_mx_rows<DT, MODE, false>), grid, dim3(256), 0, s, g, R, C, base, oc, os, tab);
  } else {
    const int64_t n_ct = (C + TC - 1) / TC, n_rt = (max_pr + TR - 1) / TR;
    // column tiles per workgroup where a table is staged (staged once; the
    // next tile's loads in flight during each tile), else 1 (measured: the
    // gathered rows of MODE 1 go faster one tile per workgroup)
    const int cpw = MODE >= 2 ? MX_T_CPW : 1;
    const int64_t n_cw = (n_ct + cpw - 1) / cpw;
    // (MODE != 1: four row tiles per span and a multiple of 8 workgroups;
    // tiles past the padded extent exit)
    dim3 grid((unsigned)(MODE == 1 ? n_cw * n_rt : xcd_grid(n_cw * ((n_rt + 3) / 4 * 4))));
    const int sfb = transpose == 2;
    if (rc) {
      if (sr)
        hipLaunchKernelGGL((k_mx_T<DT, MODE, true, true>), grid, dim3(MXT), 0, s, g, R, C, off, offp, G, max_pr, n_ct,
                           cpw, base, sfb, oc, os, tab, rc, rs);
      else
        hipLaunchKernelGGL((k_mx_T<DT, MODE, false, true>), grid, dim3(MXT), 0, s, g, R, C, off, offp, G, max_pr, n_ct,
                           cpw, base, sfb, oc, os, tab, rc, rs);
    } else if (sr) {
      hipLaunchKernelGGL((k_mx_T<DT, MODE, true, false>), grid, dim3(MXT), 0, s, g, R, C, off, offp, G, max_pr, n_ct,
                         cpw, base, sfb, oc, os, tab, nullptr, nullptr);
    } else {
      hipLaunchKernelGGL((k_mx_T<DT, MODE, false, false>), grid, dim3(MXT), 0, s, g, R, C, off, offp, G, max_pr, n_ct,
                         cpw, base, sfb, oc, os, tab, nullptr, nullptr);
    }
  }
}

}  // namespace moe4

using namespace moe4;

extern "C" int mxfp8_requant_sr_T(const uint8_t* codes, const uint8_t* sf, const float* ts, int ts_per_group,
                                  int64_t rows, int64_t cols, const int32_t* group_row_off,
                                  const int32_t* group_off_pad, int32_t n_groups, int64_t max_padded_rows,
                                  uint64_t seed, uint32_t stream_id, int sf_layout, uint8_t* out_codes,
                                  uint8_t* out_sf, void* stream) {
  MOE4_REQUIRE(rows >= 0 && cols > 0 && cols % 32 == 0, MOE4_EINVAL, "mxfp8_requant_sr_T: cols must be a positive multiple of 32");
  MOE4_REQUIRE(n_groups >= 1 && group_row_off && group_off_pad, MOE4_EINVAL, "mxfp8_requant_sr_T: group offsets required");
  MOE4_REQUIRE(max_padded_rows >= 0 && max_padded_rows % 32 == 0, MOE4_EINVAL,
               "mxfp8_requant_sr_T: max_padded_rows must be a multiple of 32");
  MOE4_REQUIRE(sf_layout == MOE4_SF_ROWS || sf_layout == MOE4_SF_BLOCKS, MOE4_EINVAL,
               "mxfp8_requant_sr_T: sf_layout must be MOE4_SF_ROWS or MOE4_SF_BLOCKS");
  MOE4_REQUIRE(codes && sf && ts && out_codes && out_sf, MOE4_EINVAL, "mxfp8_requant_sr_T: NULL pointer");
  MOE4_REQUIRE(aligned16(codes) && aligned16(out_codes), MOE4_EALIGN, "mxfp8_requant_sr_T: misaligned pointer");
  if (max_padded_rows == 0) return MOE4_OK;
  const int64_t n_ct = (cols + rq::COLS - 1) / rq::COLS, n_rt = (max_padded_rows + rq::ROWS - 1) / rq::ROWS;
  MOE4_REQUIRE(n_ct * n_rt < (int64_t)1 << 31, MOE4_EINVAL, "mxfp8_requant_sr_T: tensor too large");
  const uint32_t base = sr_base_key(seed, stream_id);
  hipLaunchKernelGGL(k_requant_T<false>, dim3((unsigned)(n_ct * n_rt)), dim3(rq::THREADS), 0, as_stream(stream), codes, sf, ts,
                     ts_per_group, cols, group_row_off, group_off_pad, n_groups, rows, max_padded_rows, n_ct, base,
                     (int)(sf_layout == MOE4_SF_BLOCKS), out_codes, out_sf);
  return check_launch("mxfp8_requant_sr_T");
}

extern "C" int mxfp8_requant_mx_sr_T(const uint8_t* codes, const uint8_t* sf, int64_t rows, int64_t cols,
                                     const int32_t* group_row_off, const int32_t* group_off_pad, int32_t n_groups,
                                     int64_t max_padded_rows, uint64_t seed, uint32_t stream_id, int sf_layout,
                                     uint8_t* out_codes, uint8_t* out_sf, void* stream) {
  MOE4_REQUIRE(rows >= 0 && cols > 0 && cols % 32 == 0, MOE4_EINVAL, "mxfp8_requant_mx_sr_T: cols must be a positive multiple of 32");
  MOE4_REQUIRE(n_groups >= 1 && group_row_off && group_off_pad, MOE4_EINVAL, "mxfp8_requant_mx_sr_T: group offsets required");
  MOE4_REQUIRE(max_padded_rows >= 0 && max_padded_rows % 32 == 0, MOE4_EINVAL,
               "mxfp8_requant_mx_sr_T: max_padded_rows must be a multiple of 32");
  MOE4_REQUIRE(sf_layout == MOE4_SF_ROWS || sf_layout == MOE4_SF_BLOCKS, MOE4_EINVAL,
               "mxfp8_requant_mx_sr_T: sf_layout must be MOE4_SF_ROWS or MOE4_SF_BLOCKS");
  MOE4_REQUIRE(codes && sf && out_codes && out_sf, MOE4_EINVAL, "mxfp8_requant_mx_sr_T: NULL pointer");
  MOE4_REQUIRE(aligned16(codes) && aligned16(out_codes), MOE4_EALIGN, "mxfp8_requant_mx_sr_T: misaligned pointer");
  if (max_padded_rows == 0) return MOE4_OK;
  const int64_t n_ct = (cols + rq::COLS - 1) / rq::COLS, n_rt = (max_padded_rows + rq::ROWS - 1) / rq::ROWS;
  MOE4_REQUIRE(n_ct * n_rt < (int64_t)1 << 31, MOE4_EINVAL, "mxfp8_requant_mx_sr_T: tensor too large");
  hipLaunchKernelGGL(k_requant_T<true>, dim3((unsigned)(n_ct * n_rt)), dim3(rq::THREADS), 0, as_stream(stream), codes,
                     sf, nullptr, 0, cols, group_row_off, group_off_pad, n_groups, rows, max_padded_rows, n_ct,
                     sr_base_key(seed, stream_id), (int)(sf_layout == MOE4_SF_BLOCKS), out_codes, out_sf);
  return check_launch("mxfp8_requant_mx_sr_T");
}

extern "C" int mxfp8_quant_requant_T(const float* x, int64_t rows, int64_t cols, int32_t n_groups, uint64_t seed,
                                     uint32_t stream_id, uint8_t* codes, uint8_t* sf, uint8_t* t_codes,
                                     uint8_t* t_sf, void* stream) {
  MOE4_REQUIRE(rows >= 0 && cols > 0 && cols % 32 == 0, MOE4_EINVAL,
               "mxfp8_quant_requant_T: cols must be a positive multiple of 32");
  MOE4_REQUIRE(n_groups >= 1 && rows % n_groups == 0 && (rows / n_groups) % 32 == 0, MOE4_EINVAL,
               "mxfp8_quant_requant_T: rows must split into n_groups equal groups of a multiple of 32 rows");
  MOE4_REQUIRE(rows == 0 || (x && codes && sf && t_codes && t_sf), MOE4_EINVAL, "mxfp8_quant_requant_T: NULL pointer");
  MOE4_REQUIRE(aligned16(x) && aligned16(codes) && aligned16(t_codes), MOE4_EALIGN,
               "mxfp8_quant_requant_T: x, codes and t_codes must be 16-byte aligned");
  if (rows == 0) return MOE4_OK;
  const int64_t grows = rows / n_groups;
  const int64_t n_ct = (cols + rq::COLS - 1) / rq::COLS, n_rt = (grows + rq::ROWS - 1) / rq::ROWS;
  const int64_t n_tiles = (int64_t)n_groups * n_rt * n_ct;
  MOE4_REQUIRE(n_tiles < ((int64_t)1 << 31), MOE4_EINVAL, "mxfp8_quant_requant_T: tensor too large");
  hipLaunchKernelGGL(k_mx_quant_requant_T, dim3((unsigned)n_tiles), dim3(rq::THREADS), 0, as_stream(stream), x, cols,
                     grows, (uint32_t)n_ct, (uint32_t)n_rt, sr_base_key(seed, stream_id), codes, sf, t_codes, t_sf);
  return check_launch("mxfp8_quant_requant_T");
}

static int mxfp8_quant_impl(const void* x, int dtype, int64_t rows, int64_t cols, const int32_t* row_map,
                            int32_t map_div, const float* row_scale, const uint16_t* dsilu_src, int pre_op,
                            int transpose, const int32_t* group_row_off, const int32_t* group_off_pad,
                            int32_t n_groups, int64_t max_padded_rows, int rnd, uint64_t seed, uint32_t stream_id,
                            uint8_t* out_codes, uint8_t* out_sf, uint8_t* row_codes, uint8_t* row_sf, void* stream) {
  MOE4_REQUIRE(dtype == MOE4_BF16 || dtype == MOE4_F32, MOE4_EINVAL, "mxfp8_quant: dtype must be BF16 or F32");
  MOE4_REQUIRE(rnd == MOE4_RNE || rnd == MOE4_SR, MOE4_EINVAL, "mxfp8_quant: rnd must be RNE or SR");
  MOE4_REQUIRE(transpose >= 0 && transpose <= 2, MOE4_EINVAL, "mxfp8_quant: transpose must be 0, 1 or 2");
  MOE4_REQUIRE(rows >= 0 && cols > 0 && cols % 32 == 0, MOE4_EINVAL, "mxfp8_quant: cols must be a positive multiple of 32");
  MOE4_REQUIRE(!(row_map && dsilu_src), MOE4_EINVAL, "mxfp8_quant: row_map and dsilu_src are exclusive");
  MOE4_REQUIRE(!row_map || map_div >= 1, MOE4_EINVAL, "mxfp8_quant: map_div >= 1");
  MOE4_REQUIRE(pre_op == MOE4_PRE_NONE || (pre_op == MOE4_PRE_SILU && dtype == MOE4_BF16 && !row_map && !dsilu_src),
               MOE4_EINVAL, "mxfp8_quant: pre_op SILU needs bf16 x and excludes row_map and dsilu_src");
  MOE4_REQUIRE(x && out_codes && out_sf, MOE4_EINVAL, "mxfp8_quant: NULL pointer");
  MOE4_REQUIRE(aligned16(x) && aligned16(out_codes) && (!dsilu_src || aligned16(dsilu_src)), MOE4_EALIGN,
               "mxfp8_quant: misaligned pointer");
  if (transpose) {
    MOE4_REQUIRE(n_groups >= 1 && group_row_off && group_off_pad, MOE4_EINVAL, "mxfp8_quant: group offsets required");
    MOE4_REQUIRE(max_padded_rows >= 0 && max_padded_rows % 32 == 0, MOE4_EINVAL,
                 "mxfp8_quant: max_padded_rows must be a multiple of 32");
  }
  hipStream_t s = as_stream(stream);
  const float* tab = nullptr;
  if (dsilu_src || pre_op == MOE4_PRE_SILU) {
    int rc = act_tables(&tab);
    if (rc) return rc;
    tab += dsilu_src ? ACT_TAB : 0;
  }
  if ((transpose ? max_padded_rows : rows) == 0) return MOE4_OK;
  if (row_codes) MOE4_REQUIRE(transpose && aligned16(row_codes) && row_sf, MOE4_EINVAL, "mxfp8_quant: row outputs");
  GradSrc g{x, dtype, row_map, map_div, row_scale, dsilu_src};
  const uint32_t base = sr_base_key(seed, stream_id);
  const bool sr = rnd == MOE4_SR;
  const int mode = row_map ? 1 : (dsilu_src ? 2 : (pre_op == MOE4_PRE_SILU ? 3 : 0));
#define MOE4_GRAD(DT, MODE)                                                                                      \
  launch_grad<DT, MODE>(transpose, sr, g, rows, cols, group_row_off, group_off_pad, n_groups, max_padded_rows, \
                        base, out_codes, out_sf, tab, s, row_codes, row_sf)
  if (dtype == MOE4_F32) {
    if (mode == 0) MOE4_GRAD(MOE4_F32, 0);
    else if (mode == 1) MOE4_GRAD(MOE4_F32, 1);
    else MOE4_GRAD(MOE4_F32, 2);
  } else {
    if (mode == 0) MOE4_GRAD(MOE4_BF16, 0);
    else if (mode == 1) MOE4_GRAD(MOE4_BF16, 1);
    else if (mode == 2) MOE4_GRAD(MOE4_BF16, 2);
    else MOE4_GRAD(MOE4_BF16, 3);
  }
#undef MOE4_GRAD
  return check_launch("mxfp8_quant");
}

extern "C" int mxfp8_quant(const void* x, int dtype, int64_t rows, int64_t cols, const int32_t* row_map,
                           int32_t map_div, const float* row_scale, const uint16_t* dsilu_src, int pre_op,
                           int transpose, const int32_t* group_row_off, const int32_t* group_off_pad,
                           int32_t n_groups, int64_t max_padded_rows, int rnd, uint64_t seed, uint32_t stream_id,
                           uint8_t* out_codes, uint8_t* out_sf, void* stream) {
  return mxfp8_quant_impl(x, dtype, rows, cols, row_map, map_div, row_scale, dsilu_src, pre_op, transpose,
                          group_row_off, group_off_pad, n_groups, max_padded_rows, rnd, seed, stream_id, out_codes,
                          out_sf, nullptr, nullptr, stream);
}

extern "C" int mxfp8_quant_rows_T(const void* x, int dtype, int64_t rows, int64_t cols, const int32_t* row_map,
                                  int32_t map_div, const float* row_scale, const uint16_t* dsilu_src,
                                  const int32_t* group_row_off, const int32_t* group_off_pad, int32_t n_groups,
                                  int64_t max_padded_rows, int rnd, uint64_t seed, uint32_t stream_id, int sf_layout,
                                  uint8_t* row_codes, uint8_t* row_sf, uint8_t* t_codes, uint8_t* t_sf,
                                  void* stream) {
  MOE4_REQUIRE(sf_layout == MOE4_SF_ROWS || sf_layout == MOE4_SF_BLOCKS, MOE4_EINVAL,
               "mxfp8_quant_rows_T: sf_layout must be MOE4_SF_ROWS or MOE4_SF_BLOCKS");
  MOE4_REQUIRE(row_codes && row_sf, MOE4_EINVAL, "mxfp8_quant_rows_T: NULL pointer");
  return mxfp8_quant_impl(x, dtype, rows, cols, row_map, map_div, row_scale, dsilu_src, MOE4_PRE_NONE,
                          sf_layout == MOE4_SF_BLOCKS ? 2 : 1, group_row_off, group_off_pad, n_groups,
                          max_padded_rows, rnd, seed, stream_id, t_codes, t_sf, row_codes, row_sf, stream);
}
