// Expert-grouped NVFP4 x NVFP4 GEMM of the forward pass (gfx950).
//
// The pages' forward runs the expert layers in NVFP4 "bolstered by a dedicated
// kernel" (agihunt.info page, "Confirmed"; fourweekmba.com page, "What
// Thinking Machines Changed").  On gfx950 the block-scaled MFMA takes E8M0
// scales per 32 values, while NVFP4 carries an E4M3 scale per 16, and an E2M1
// value times an E4M3 scale needs up to 6 significant bits, more than any
// FP8/FP6 operand has.  The exact path is therefore: dequantise each operand
// block to f16 exactly while staging it into LDS (hardware FP4 -> f16 convert
// by the scale's power of two, then one packed f16 multiply by the scale's
// mantissa 1.m; |q*sc| lies in [2**-10, 2688], all normal f16), and run f16
// MFMA 32x32x16 with float32 accumulation.  Tensor scales S_a * S_b[e] are
// applied in the epilogue.
//
// C[rows of e] = A[rows of e] . B[e]^T; A [M_total, K], B [E, N, K], both
// with K contiguous; rows of A grouped by expert_off.  Tile BM x 256 x 64,
// 256 threads as 2 x 2 waves of (BM/2) x 128; double-buffered LDS (f16 rows
// padded to 144 bytes), one barrier per K slab: the next slab's NVFP4 codes
// are fetched into registers before the current slab's MFMAs and dequantised
// into the other LDS buffer after them.  The epilogue stages the tile through
// LDS for row-contiguous 16-byte (f32) or 8-byte (bf16) stores.
#include <stdlib.h>

#include "gemm_common.h"
#include "moe4_internal.h"

namespace moe4 {

namespace fwd {
constexpr int BK = 64;
constexpr int LDS_STRIDE = BK + 8;  // halfs per LDS row (144 bytes)
constexpr int THREADS = 256;
}  // namespace fwd

// Register staging of one slab: ROWS rows x 64 elements (32 code bytes and 4
// scale bytes per row); thread t holds rows t/2 + 128 j, half t % 2 (16 code
// bytes, 2 scale bytes).
template <int ROWS>
struct Fp4Slab {
  u32x4 q[ROWS / 128];
  uint32_t s[ROWS / 128];
};

template <int ROWS>
__device__ inline void load_fp4_slab(Fp4Slab<ROWS>& f, const uint8_t* codes, const uint8_t* sf, int64_t row0,
                                     int64_t row_end, int64_t K, int64_t k0) {
  const int t = threadIdx.x, half = t & 1;
#pragma unroll
  for (int j = 0; j < ROWS / 128; ++j) {
    // rows past the valid range are clamped to the last valid row: their
    // outputs are never stored, so every load is unconditional
    int64_t row = row0 + (t >> 1) + 128 * j;
    row = row < row_end ? row : row_end - 1;
    f.q[j] = *reinterpret_cast<const u32x4*>(codes + row * (K / 2) + k0 / 2 + half * 16);
    f.s[j] = *reinterpret_cast<const uint16_t*>(sf + row * (K / 16) + k0 / 16 + half * 2);
  }
}

// Exact f16 values of 32 elements (two 16-element blocks), written to LDS.
__device__ inline void dequant32_to_lds(u32x4 q, uint32_t s, _Float16* dst) {
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    const float scf = e4m3_to_f32((s >> (8 * hb)) & 0xFFu);
    const _Float16 mh = (_Float16)mant_factor(scf);  // 1.m, exact in f16
    const f16x2 m2 = {mh, mh};
    uint32_t w[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t word = q[hb * 2 + (j >> 2)];
      const uint32_t byte = (word >> (8 * (j & 3))) & 0xFFu;
      f16x2 h = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(byte, scf, 0);  // q * 2**floor(log2 sc)
      h = h * m2;                                                       // exact q * sc
      w[j] = __builtin_bit_cast(uint32_t, h);
    }
    u32x4* d = reinterpret_cast<u32x4*>(dst + hb * 16);
    d[0] = u32x4{w[0], w[1], w[2], w[3]};
    d[1] = u32x4{w[4], w[5], w[6], w[7]};
  }
}

template <int ROWS>
__device__ inline void store_fp4_slab(const Fp4Slab<ROWS>& f, _Float16* lds) {
  const int t = threadIdx.x, half = t & 1;
#pragma unroll
  for (int j = 0; j < ROWS / 128; ++j)
    dequant32_to_lds(f.q[j], f.s[j], lds + ((t >> 1) + 128 * j) * fwd::LDS_STRIDE + half * 32);
}

template <bool OUT_BF16, int BM, int BN, int MINB>
__global__ void __launch_bounds__(fwd::THREADS, MINB) k_gemm_fwd(const uint8_t* __restrict__ a_codes,
                                                              const uint8_t* __restrict__ a_sf,
                                                              const float* __restrict__ a_ts, int a_ts_per_group,
                                                              const uint8_t* __restrict__ b_codes,
                                                              const uint8_t* __restrict__ b_sf,
                                                              const float* __restrict__ b_ts,
                                                              const int32_t* __restrict__ off, int E, int64_t M_total,
                                                              int64_t N, int64_t K, int64_t n_ntiles,
                                                              void* __restrict__ c) {
  using namespace fwd;
  constexpr int WM = BM / 2, MI = WM / 32, WN = BN / 2, NJ = WN / 32;
  constexpr int A_H = BM * LDS_STRIDE, B_H = BN * LDS_STRIDE;  // halfs
  constexpr int STAGE = A_H + B_H;
  __shared__ __attribute__((aligned(16))) _Float16 smem[2 * STAGE];

  const int64_t n_all = n_ntiles * ((M_total + BM - 1) / BM + E);
  const int64_t tile = xcd_tile(blockIdx.x, n_all);
  if (tile >= n_all) return;
  const int64_t nt = tile % n_ntiles;
  int e;
  int64_t mt;
  if (!find_m_tile(off, E, BM, tile / n_ntiles, e, mt)) return;
  const int64_t row0 = (int64_t)off[e] + mt * BM;
  const int64_t row_end = (int64_t)off[e + 1] < M_total ? (int64_t)off[e + 1] : M_total;
  const int64_t n0 = nt * BN;
  const uint8_t* bcodes = b_codes + (int64_t)e * N * (K / 2);
  const uint8_t* bsf = b_sf + (int64_t)e * N * (K / 16);
  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63;
  const int wm = (w >> 1) * WM, wn = (w & 1) * WN;
  const int g = l >> 5, li = l & 31;

  f32x16 acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = f32x16{};

  // Two register sets keep two slabs in flight: the codes of slab it+2 are
  // loaded before slab it's MFMAs and dequantised into LDS one slab later.
  Fp4Slab<BM> fa0, fa1;
  Fp4Slab<BN> fb0, fb1;
  const int64_t nk = K / BK;
  auto fetch = [&](Fp4Slab<BM>& fa, Fp4Slab<BN>& fb, int64_t k0) {
    load_fp4_slab<BM>(fa, a_codes, a_sf, row0, row_end, K, k0);
    load_fp4_slab<BN>(fb, bcodes, bsf, n0, N, K, k0);
  };
  auto stash = [&](const Fp4Slab<BM>& fa, const Fp4Slab<BN>& fb, _Float16* st) {
    store_fp4_slab<BM>(fa, st);
    store_fp4_slab<BN>(fb, st + A_H);
  };
  auto compute = [&](const _Float16* la) {
    const _Float16* lb = la + A_H;
#pragma unroll
    for (int kk = 0; kk < BK; kk += 16) {
      f16x8 bv[NJ];
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        bv[j] = *reinterpret_cast<const f16x8*>(lb + (wn + j * 32 + li) * LDS_STRIDE + kk + g * 8);
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        const f16x8 av = *reinterpret_cast<const f16x8*>(la + (wm + i * 32 + li) * LDS_STRIDE + kk + g * 8);
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, bv[j], acc[i][j], 0, 0, 0);
      }
    }
  };
  _Float16* buf0 = smem;
  _Float16* buf1 = smem + STAGE;
  fetch(fa0, fb0, 0);
  stash(fa0, fb0, buf0);
  if (nk > 1) fetch(fa1, fb1, BK);
  __syncthreads();
  for (int64_t it = 0; it < nk; it += 2) {
    if (it + 2 < nk) fetch(fa0, fb0, (it + 2) * BK);
    compute(buf0);
    if (it + 1 < nk) stash(fa1, fb1, buf1);
    __syncthreads();
    if (it + 1 >= nk) break;
    if (it + 3 < nk) fetch(fa1, fb1, (it + 3) * BK);
    compute(buf1);
    if (it + 2 < nk) stash(fa0, fb0, buf0);
    __syncthreads();
  }
  // Epilogue: 32-row bands of each wave's tile through LDS, scaled by S_a*S_b.
  const float sab = a_ts[a_ts_per_group ? e : 0] * b_ts[e];
  constexpr int BS = WN + 4;
  static_assert(4 * 32 * BS * 4 <= 2 * STAGE * 2, "epilogue band does not fit");
  float* band = reinterpret_cast<float*>(smem) + w * (32 * BS);
#pragma unroll
  for (int i = 0; i < MI; ++i) {
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) band[((v >> 2) * 8 + g * 4 + (v & 3)) * BS + j * 32 + li] = acc[i][j][v] * sab;
    __builtin_amdgcn_wave_barrier();
    constexpr int QPR = WN / 4;
#pragma unroll
    for (int q = 0; q < 32 * QPR / 64; ++q) {
      const int idx = q * 64 + l;
      const int rr = idx / QPR, cq = idx % QPR;
      const int64_t row = row0 + wm + i * 32 + rr;
      const int64_t col = n0 + wn + cq * 4;
      if (row < row_end && col < N) {
        f32x4 v = *reinterpret_cast<const f32x4*>(band + rr * BS + cq * 4);
        if (OUT_BF16) {
          u32x2 o = {f32_to_bf16_bits(v[0]) | (f32_to_bf16_bits(v[1]) << 16),
                     f32_to_bf16_bits(v[2]) | (f32_to_bf16_bits(v[3]) << 16)};
          *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(c) + row * N + col) = o;
        } else {
          __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(static_cast<float*>(c) + row * N + col));
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
}

template <bool OUT_BF16, int BM, int BN, int MINB>
static void launch_fwd_t(hipStream_t s, const uint8_t* ac, const uint8_t* as, const float* ats, int apg,
                         const uint8_t* bc, const uint8_t* bs, const float* bts, const int32_t* off, int E, int64_t M,
                         int64_t N, int64_t K, void* c) {
  const int64_t n_nt = (N + BN - 1) / BN;
  const int64_t n_mt = (M + BM - 1) / BM + E;  // upper bound of the grouped m-tiles
  hipLaunchKernelGGL((k_gemm_fwd<OUT_BF16, BM, BN, MINB>), dim3((unsigned)xcd_grid(n_nt * n_mt)), dim3(fwd::THREADS), 0, s, ac,
                     as, ats, apg, bc, bs, bts, off, E, M, N, K, n_nt, c);
}

// Configuration choice (MOE4_FWD_TILE overrides, for tuning): 0 = 128x128
// (2 blocks/CU), 1 = 256x256, 2 = 128x256.
static int fwd_tile_choice() {
  static int v = [] {
    const char* e = getenv("MOE4_FWD_TILE");
    return e ? atoi(e) : 0;
  }();
  return v;
}

template <bool OUT_BF16>
static void launch_fwd(hipStream_t s, const uint8_t* ac, const uint8_t* as, const float* ats, int apg,
                       const uint8_t* bc, const uint8_t* bs, const float* bts, const int32_t* off, int E, int64_t M,
                       int64_t N, int64_t K, void* c) {
  switch (fwd_tile_choice()) {
    case 1: launch_fwd_t<OUT_BF16, 256, 256, 1>(s, ac, as, ats, apg, bc, bs, bts, off, E, M, N, K, c); break;
    case 2: launch_fwd_t<OUT_BF16, 128, 256, 1>(s, ac, as, ats, apg, bc, bs, bts, off, E, M, N, K, c); break;
    default: launch_fwd_t<OUT_BF16, 128, 128, 2>(s, ac, as, ats, apg, bc, bs, bts, off, E, M, N, K, c); break;
  }
}

}  // namespace moe4

using namespace moe4;

extern "C" int moe_grouped_gemm_fwd(const uint8_t* a_codes, const uint8_t* a_sf, const float* a_ts, int a_ts_per_group,
                                    const uint8_t* b_codes, const uint8_t* b_sf, const float* b_ts,
                                    const int32_t* expert_off, int32_t E, int64_t M_total, int64_t N, int64_t K,
                                    void* c, int c_dtype, void* stream) {
  MOE4_REQUIRE(E >= 1 && M_total >= 0 && N > 0 && K > 0, MOE4_EINVAL, "moe_grouped_gemm_fwd: bad sizes");
  MOE4_REQUIRE(K % 64 == 0 && N % 32 == 0, MOE4_EINVAL, "moe_grouped_gemm_fwd: need K % 64 == 0 and N % 32 == 0");
  MOE4_REQUIRE(c_dtype == MOE4_BF16 || c_dtype == MOE4_F32, MOE4_EINVAL, "moe_grouped_gemm_fwd: c_dtype");
  MOE4_REQUIRE(a_ts && b_codes && b_sf && b_ts && expert_off, MOE4_EINVAL, "moe_grouped_gemm_fwd: NULL pointer");
  MOE4_REQUIRE(M_total == 0 || (a_codes && a_sf && c), MOE4_EINVAL, "moe_grouped_gemm_fwd: NULL pointer");
  MOE4_REQUIRE(aligned16(a_codes) && aligned16(b_codes) && aligned16(c), MOE4_EALIGN,
               "moe_grouped_gemm_fwd: misaligned pointer");
  if (M_total == 0) return MOE4_OK;
  MOE4_REQUIRE(((N + 127) / 128) * ((M_total + 127) / 128 + E) < ((int64_t)1 << 31), MOE4_EINVAL,
               "moe_grouped_gemm_fwd: too large");
  hipStream_t s = as_stream(stream);
  if (c_dtype == MOE4_BF16)
    launch_fwd<true>(s, a_codes, a_sf, a_ts, a_ts_per_group, b_codes, b_sf, b_ts, expert_off, E, M_total, N, K, c);
  else
    launch_fwd<false>(s, a_codes, a_sf, a_ts, a_ts_per_group, b_codes, b_sf, b_ts, expert_off, E, M_total, N, K, c);
  return check_launch("moe_grouped_gemm_fwd");
}
