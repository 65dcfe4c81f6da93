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
// with K contiguous; rows of A grouped by expert_off.  Tile 128 x 128 x 64,
// 256 threads as 2 x 2 waves of 64 x 64; the next K-slab's codes are fetched
// into registers while the current slab's MFMAs run.
#include "gemm_common.h"
#include "moe4_internal.h"

namespace moe4 {

namespace fwd {
constexpr int BM = 128, BN = 128, BK = 64;
constexpr int LDS_STRIDE = BK + 8;  // halfs per LDS row (pad: spread banks)
constexpr int THREADS = 256;
}  // namespace fwd

// One thread's share of a K-slab: 32 elements (16 code bytes) + 2 scale bytes
// of one row.
struct Fp4Frag {
  u32x4 q;
  uint32_t s;  // two E4M3 bytes
};

__device__ inline Fp4Frag load_fp4_frag(const uint8_t* codes, const uint8_t* sf, int64_t row, bool valid, int64_t K,
                                        int64_t k0, int half) {
  Fp4Frag f;
  if (valid) {
    f.q = *reinterpret_cast<const u32x4*>(codes + row * (K / 2) + k0 / 2 + half * 16);
    const uint8_t* sp = sf + row * (K / 16) + k0 / 16 + half * 2;
    f.s = (uint32_t)sp[0] | ((uint32_t)sp[1] << 8);
  } else {
    f.q = u32x4{0u, 0u, 0u, 0u};
    f.s = 0u;
  }
  return f;
}

// Exact f16 values of the 32 elements, written to LDS (4 x 16 bytes).
__device__ inline void store_fp4_frag_f16(const Fp4Frag& f, _Float16* dst) {
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {  // two 16-element blocks, one scale each
    const float scf = e4m3_to_f32((f.s >> (8 * hb)) & 0xFFu);
    const _Float16 mh = (_Float16)mant_factor(scf);  // 1.m, exact in f16
    const f16x2 m2 = {mh, mh};
    uint32_t w[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {  // 8 bytes = 16 elements
      const uint32_t word = f.q[hb * 2 + (j >> 2)];
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

template <bool OUT_BF16>
__global__ void __launch_bounds__(fwd::THREADS) k_gemm_fwd(const uint8_t* __restrict__ a_codes,
                                                           const uint8_t* __restrict__ a_sf,
                                                           const float* __restrict__ a_ts, int a_ts_per_group,
                                                           const uint8_t* __restrict__ b_codes,
                                                           const uint8_t* __restrict__ b_sf,
                                                           const float* __restrict__ b_ts,
                                                           const int32_t* __restrict__ off, int E, int64_t M_total,
                                                           int64_t N, int64_t K, int64_t n_ntiles,
                                                           void* __restrict__ c) {
  using namespace fwd;
  __shared__ __attribute__((aligned(16))) _Float16 la[BM * LDS_STRIDE];
  __shared__ __attribute__((aligned(16))) _Float16 lb[BN * LDS_STRIDE];
  const int64_t nt = blockIdx.x % n_ntiles;
  const int64_t mt_flat = blockIdx.x / n_ntiles;
  int e;
  int64_t mt;
  if (!find_m_tile(off, E, BM, mt_flat, e, mt)) return;
  const int64_t row0 = (int64_t)off[e] + mt * BM;
  const int64_t row_end = (int64_t)off[e + 1] < M_total ? (int64_t)off[e + 1] : M_total;
  const int64_t n0 = nt * BN;
  const int tid = threadIdx.x;
  const int lrow = tid >> 1, half = tid & 1;
  const bool a_ok = row0 + lrow < row_end;
  const bool b_ok = n0 + lrow < N;
  const uint8_t* bcodes = b_codes + (int64_t)e * N * (K / 2);
  const uint8_t* bsf = b_sf + (int64_t)e * N * (K / 16);

  const int w = tid >> 6, l = tid & 63;
  const int wm = (w >> 1) * 64, wn = (w & 1) * 64;
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  Fp4Frag fa = load_fp4_frag(a_codes, a_sf, row0 + lrow, a_ok, K, 0, half);
  Fp4Frag fb = load_fp4_frag(bcodes, bsf, n0 + lrow, b_ok, K, 0, half);
  for (int64_t k0 = 0; k0 < K; k0 += BK) {
    __syncthreads();  // previous slab's MFMA reads are done
    store_fp4_frag_f16(fa, la + lrow * LDS_STRIDE + half * 32);
    store_fp4_frag_f16(fb, lb + lrow * LDS_STRIDE + half * 32);
    __syncthreads();
    if (k0 + BK < K) {  // prefetch the next slab into registers
      fa = load_fp4_frag(a_codes, a_sf, row0 + lrow, a_ok, K, k0 + BK, half);
      fb = load_fp4_frag(bcodes, bsf, n0 + lrow, b_ok, K, k0 + BK, half);
    }
#pragma unroll
    for (int kk = 0; kk < BK; kk += 16) {
      f16x8 av[2], bv[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        av[i] = *reinterpret_cast<const f16x8*>(la + (wm + i * 32 + (l & 31)) * LDS_STRIDE + kk + (l >> 5) * 8);
        bv[i] = *reinterpret_cast<const f16x8*>(lb + (wn + i * 32 + (l & 31)) * LDS_STRIDE + kk + (l >> 5) * 8);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[i], bv[j], acc[i][j], 0, 0, 0);
    }
  }
  const float sab = a_ts[a_ts_per_group ? e : 0] * b_ts[e];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t col = n0 + wn + j * 32 + (l & 31);
      if (col >= N) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t row = row0 + wm + i * 32 + (v >> 2) * 8 + (l >> 5) * 4 + (v & 3);
        if (row >= row_end) continue;
        const float val = acc[i][j][v] * sab;
        if (OUT_BF16)
          static_cast<uint16_t*>(c)[row * N + col] = (uint16_t)f32_to_bf16_bits(val);
        else
          static_cast<float*>(c)[row * N + col] = val;
      }
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
  const int64_t n_nt = (N + fwd::BN - 1) / fwd::BN;
  const int64_t n_mt = (M_total + fwd::BM - 1) / fwd::BM + E;  // upper bound of the grouped m-tiles
  MOE4_REQUIRE(n_nt * n_mt < ((int64_t)1 << 31), MOE4_EINVAL, "moe_grouped_gemm_fwd: too large");
  dim3 grid((unsigned)(n_nt * n_mt));
  hipStream_t s = as_stream(stream);
  if (c_dtype == MOE4_BF16)
    hipLaunchKernelGGL((k_gemm_fwd<true>), grid, dim3(fwd::THREADS), 0, s, a_codes, a_sf, a_ts, a_ts_per_group, b_codes,
                       b_sf, b_ts, expert_off, E, M_total, N, K, n_nt, c);
  else
    hipLaunchKernelGGL((k_gemm_fwd<false>), grid, dim3(fwd::THREADS), 0, s, a_codes, a_sf, a_ts, a_ts_per_group,
                       b_codes, b_sf, b_ts, expert_off, E, M_total, N, K, n_nt, c);
  return check_launch("moe_grouped_gemm_fwd");
}
