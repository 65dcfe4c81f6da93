// Expert-grouped MXFP8 GEMMs of the backward pass (gfx950): dgrad (rows
// grouped by expert) and wgrad (the contraction runs over each expert's
// padded token range).
//
// The pages run backpropagation in MXFP8 (agihunt.info page, "Confirmed";
// lhc.media page, paragraph on the backward pass).  MXFP8's E8M0 scale per 32
// values along the contraction is exactly what gfx950's block-scaled MFMA
// (v_mfma_scale_f32_32x32x64_f8f6f4) applies, so both operands feed the
// matrix cores natively: exact products, float32 accumulation.
//
// Operand layout of the 32x32x64 scaled MFMA (measured on gfx950): lane l
// (g = l / 32, i = l % 32) holds row i's bytes k in [16g, 16g+16) and
// [32+16g, 32+16g+16) of the 64-wide K chunk, and supplies the scale of row i,
// K block g.  Tile 128 x 128 x 128 bytes, 256 threads as 2 x 2 waves of
// 64 x 64; next slab prefetched into registers during the MFMAs.
#include "gemm_common.h"
#include "moe4_internal.h"

namespace moe4 {

namespace bwd {
constexpr int BM = 128, BN = 128, BK = 128;
constexpr int LDS_STRIDE = BK + 16;  // bytes per LDS row
constexpr int THREADS = 256;
}  // namespace bwd

struct Fp8Frag {
  u32x4 q[4];  // 64 bytes
  uint32_t s;  // 2 scale bytes
};

// Row `row` of an MXFP8 operand with row stride ld (bytes) and scale row
// stride ld/32; 64 bytes at k0 + half*64, masked to k < klen.
__device__ inline Fp8Frag load_fp8_frag(const uint8_t* codes, const uint8_t* sf, int64_t row, bool valid, int64_t ld,
                                        int64_t klen, int64_t k0, int half) {
  Fp8Frag f;
  const int64_t kb = k0 + half * 64;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const bool ok = valid && kb + 16 * c < klen;
    f.q[c] = ok ? *reinterpret_cast<const u32x4*>(codes + row * ld + kb + 16 * c) : u32x4{0u, 0u, 0u, 0u};
  }
  f.s = 0u;
  if (valid) {
    const uint8_t* sp = sf + row * (ld / 32) + kb / 32;
    if (kb < klen) f.s |= (uint32_t)sp[0];
    if (kb + 32 < klen) f.s |= (uint32_t)sp[1] << 8;
  }
  return f;
}

__device__ inline void store_fp8_frag(const Fp8Frag& f, uint8_t* dst_row, uint8_t* dst_scale_row, int half) {
  u32x4* d = reinterpret_cast<u32x4*>(dst_row + half * 64);
#pragma unroll
  for (int c = 0; c < 4; ++c) d[c] = f.q[c];
  dst_scale_row[half * 2] = (uint8_t)(f.s & 0xFFu);
  dst_scale_row[half * 2 + 1] = (uint8_t)(f.s >> 8);
}

// MODE 0: dgrad (A rows grouped by expert_off, B [E][N][K], C [M_total][N]);
// MODE 1: wgrad (per expert e: A_e [N1][P_e], B_e [N2][P_e], C = dw[e]).
template <int MODE>
__global__ void __launch_bounds__(bwd::THREADS) k_gemm_mx(const uint8_t* __restrict__ a_codes,
                                                          const uint8_t* __restrict__ a_sf,
                                                          const uint8_t* __restrict__ b_codes,
                                                          const uint8_t* __restrict__ b_sf,
                                                          const int32_t* __restrict__ off, int E, int64_t M1,
                                                          int64_t N, int64_t K, int64_t n_ntiles, int64_t n_mtiles,
                                                          float* __restrict__ c, float beta) {
  using namespace bwd;
  __shared__ __attribute__((aligned(16))) uint8_t la[BM * LDS_STRIDE];
  __shared__ __attribute__((aligned(16))) uint8_t lb[BN * LDS_STRIDE];
  __shared__ __attribute__((aligned(16))) uint8_t las[BM * 4];
  __shared__ __attribute__((aligned(16))) uint8_t lbs[BN * 4];
  const int64_t nt = blockIdx.x % n_ntiles;
  int64_t row0, row_end, klen, lda, ldc;
  const uint8_t *A, *As, *B, *Bs;
  float* C;
  if (MODE == 0) {
    int e;
    int64_t mt;
    if (!find_m_tile(off, E, BM, blockIdx.x / n_ntiles, e, mt)) return;
    row0 = (int64_t)off[e] + mt * BM;
    row_end = (int64_t)off[e + 1] < M1 ? (int64_t)off[e + 1] : M1;  // M1 = M_total here
    klen = K;
    lda = K;
    A = a_codes;
    As = a_sf;
    B = b_codes + (int64_t)e * N * K;
    Bs = b_sf + (int64_t)e * N * (K / 32);
    C = c;
    ldc = N;
  } else {
    const int64_t rest = blockIdx.x / n_ntiles;
    const int e = (int)(rest / n_mtiles);
    const int64_t mt = rest % n_mtiles;
    if (e >= E) return;
    const int64_t p0 = off[e];
    klen = (int64_t)off[e + 1] - p0;  // padded token count (multiple of 32)
    row0 = mt * BM;
    row_end = M1;
    lda = klen;
    A = a_codes + M1 * p0;
    As = a_sf + M1 * p0 / 32;
    B = b_codes + N * p0;
    Bs = b_sf + N * p0 / 32;
    C = c + (int64_t)e * M1 * N;
    ldc = N;
    if (klen == 0 && beta != 0.0f) return;  // nothing to add
  }
  const int64_t n0 = nt * BN;
  const int tid = threadIdx.x;
  const int lrow = tid >> 1, half = tid & 1;
  const bool a_ok = row0 + lrow < row_end;
  const bool b_ok = n0 + lrow < N;
  const int w = tid >> 6, l = tid & 63;
  const int wm = (w >> 1) * 64, wn = (w & 1) * 64;
  const int g = l >> 5, li = l & 31;
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  Fp8Frag fa, fb;
  if (klen > 0) {
    fa = load_fp8_frag(A, As, row0 + lrow, a_ok, lda, klen, 0, half);
    fb = load_fp8_frag(B, Bs, n0 + lrow, b_ok, lda, klen, 0, half);
  }
  for (int64_t k0 = 0; k0 < klen; k0 += BK) {
    __syncthreads();
    store_fp8_frag(fa, la + lrow * LDS_STRIDE, las + lrow * 4, half);
    store_fp8_frag(fb, lb + lrow * LDS_STRIDE, lbs + lrow * 4, half);
    __syncthreads();
    if (k0 + BK < klen) {
      fa = load_fp8_frag(A, As, row0 + lrow, a_ok, lda, klen, k0 + BK, half);
      fb = load_fp8_frag(B, Bs, n0 + lrow, b_ok, lda, klen, k0 + BK, half);
    }
#pragma unroll
    for (int kc = 0; kc < BK; kc += 64) {
      i32x8 av[2], bv[2];
      int sa[2], sb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const uint8_t* pa = la + (wm + i * 32 + li) * LDS_STRIDE + kc + 16 * g;
        const uint8_t* pb = lb + (wn + i * 32 + li) * LDS_STRIDE + kc + 16 * g;
        i32x4 a0 = *reinterpret_cast<const i32x4*>(pa), a1 = *reinterpret_cast<const i32x4*>(pa + 32);
        i32x4 b0 = *reinterpret_cast<const i32x4*>(pb), b1 = *reinterpret_cast<const i32x4*>(pb + 32);
        av[i] = i32x8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
        bv[i] = i32x8{b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
        sa[i] = las[(wm + i * 32 + li) * 4 + kc / 32 + g];
        sb[i] = lbs[(wn + i * 32 + li) * 4 + kc / 32 + g];
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av[i], bv[j], acc[i][j], 0, 0, 0, sa[i], 0,
                                                                      sb[j]);
    }
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t col = n0 + wn + j * 32 + li;
      if (col >= N) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t row = row0 + wm + i * 32 + (v >> 2) * 8 + g * 4 + (v & 3);
        if (row >= row_end) continue;
        float* p = C + row * ldc + col;
        if (MODE == 1 && beta != 0.0f) *p = *p + acc[i][j][v];
        else *p = acc[i][j][v];
      }
    }
}

}  // namespace moe4

using namespace moe4;

extern "C" int moe_grouped_gemm_bwd_dgrad(const uint8_t* a_codes, const uint8_t* a_sf, const uint8_t* b_codes,
                                          const uint8_t* b_sf, const int32_t* expert_off, int32_t E, int64_t M_total,
                                          int64_t N, int64_t K, float* c, void* stream) {
  MOE4_REQUIRE(E >= 1 && M_total >= 0 && N > 0 && K > 0 && K % 32 == 0 && N % 32 == 0, MOE4_EINVAL,
               "moe_grouped_gemm_bwd_dgrad: need K % 32 == 0 and N % 32 == 0");
  MOE4_REQUIRE(b_codes && b_sf && expert_off, MOE4_EINVAL, "moe_grouped_gemm_bwd_dgrad: NULL pointer");
  MOE4_REQUIRE(M_total == 0 || (a_codes && a_sf && c), MOE4_EINVAL, "moe_grouped_gemm_bwd_dgrad: NULL pointer");
  MOE4_REQUIRE(aligned16(a_codes) && aligned16(b_codes) && aligned16(c), MOE4_EALIGN,
               "moe_grouped_gemm_bwd_dgrad: misaligned pointer");
  if (M_total == 0) return MOE4_OK;
  const int64_t n_nt = (N + bwd::BN - 1) / bwd::BN;
  const int64_t n_mt = (M_total + bwd::BM - 1) / bwd::BM + E;
  MOE4_REQUIRE(n_nt * n_mt < ((int64_t)1 << 31), MOE4_EINVAL, "moe_grouped_gemm_bwd_dgrad: too large");
  hipLaunchKernelGGL((k_gemm_mx<0>), dim3((unsigned)(n_nt * n_mt)), dim3(bwd::THREADS), 0, as_stream(stream), a_codes,
                     a_sf, b_codes, b_sf, expert_off, E, M_total, N, K, n_nt, n_mt, c, 0.0f);
  return check_launch("moe_grouped_gemm_bwd_dgrad");
}

extern "C" int moe_grouped_gemm_bwd_wgrad(const uint8_t* a_codes, const uint8_t* a_sf, const uint8_t* b_codes,
                                          const uint8_t* b_sf, const int32_t* expert_off_pad, int32_t E, int64_t N1,
                                          int64_t N2, float* dw, float beta, void* stream) {
  MOE4_REQUIRE(E >= 1 && N1 > 0 && N2 > 0 && N1 % 32 == 0 && N2 % 32 == 0, MOE4_EINVAL,
               "moe_grouped_gemm_bwd_wgrad: need N1 % 32 == 0 and N2 % 32 == 0");
  MOE4_REQUIRE(beta == 0.0f || beta == 1.0f, MOE4_EINVAL, "moe_grouped_gemm_bwd_wgrad: beta must be 0 or 1");
  MOE4_REQUIRE(a_codes && a_sf && b_codes && b_sf && expert_off_pad && dw, MOE4_EINVAL,
               "moe_grouped_gemm_bwd_wgrad: NULL pointer");
  MOE4_REQUIRE(aligned16(a_codes) && aligned16(b_codes) && aligned16(dw), MOE4_EALIGN,
               "moe_grouped_gemm_bwd_wgrad: misaligned pointer");
  const int64_t n_nt = (N2 + bwd::BN - 1) / bwd::BN;
  const int64_t n_mt = (N1 + bwd::BM - 1) / bwd::BM;
  MOE4_REQUIRE(n_nt * n_mt * E < ((int64_t)1 << 31), MOE4_EINVAL, "moe_grouped_gemm_bwd_wgrad: too large");
  hipLaunchKernelGGL((k_gemm_mx<1>), dim3((unsigned)(n_nt * n_mt * E)), dim3(bwd::THREADS), 0, as_stream(stream),
                     a_codes, a_sf, b_codes, b_sf, expert_off_pad, E, N1, N2, (int64_t)0, n_nt, n_mt, dw, beta);
  return check_launch("moe_grouped_gemm_bwd_wgrad");
}

extern "C" int moe_grouped_gemm_bwd(const uint8_t* dy_codes, const uint8_t* dy_sf, const uint8_t* wT_codes,
                                    const uint8_t* wT_sf, const uint8_t* dyT_codes, const uint8_t* dyT_sf,
                                    const uint8_t* xT_codes, const uint8_t* xT_sf, const int32_t* expert_off,
                                    const int32_t* expert_off_pad, int32_t E, int64_t M_total, int64_t Nin,
                                    int64_t Nout, float* dx, float* dw, float beta, void* stream) {
  int rc = moe_grouped_gemm_bwd_dgrad(dy_codes, dy_sf, wT_codes, wT_sf, expert_off, E, M_total, Nin, Nout, dx, stream);
  if (rc) return rc;
  return moe_grouped_gemm_bwd_wgrad(dyT_codes, dyT_sf, xT_codes, xT_sf, expert_off_pad, E, Nout, Nin, dw, beta, stream);
}
