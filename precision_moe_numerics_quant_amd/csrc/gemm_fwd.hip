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

#include "act.h"
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

// ------------------------------------------------ direct-to-LDS variant
// K % 256 == 0.  256 x 256 tile, 4 waves of 128 x 128, K slabs of 256
// elements: 128 code bytes and 16 scale bytes per row, both fetched straight
// into LDS (each load instruction of a wave fills 1 KB: 8 whole 128-byte
// rows of codes, or 64 rows of scales), two LDS buffers, one barrier per
// slab.  Each wave dequantises its own fragments in registers right before
// the f16 MFMAs (hardware FP4 -> f16 by the scale's power of two, times the
// mantissa 1.m: exact), so LDS holds the 4-bit data only.  The slab's 256 K
// positions are assigned to MFMA steps in an order that both operands share
// (a dot product does not depend on it): lane half g takes elements
// 128 g + 8 ks .. 128 g + 8 ks + 7 at step ks, i.e. the contiguous bytes
// 64 g .. 64 g + 63 of its row over the slab's 16 steps, and the 8 scale bytes
// 8 g .. 8 g + 7.  Code rows keep their 16-byte chunks XOR-swizzled by
// (row >> 1) & 7 (applied through the fetched global address) so that 16
// lanes reading one chunk of 16 consecutive rows hit distinct bank groups.
namespace fdma {
constexpr int BKE = 256, RB = BKE / 2, NT = 256;  // RB: code bytes per row and slab
__device__ inline int swz(int row, int c) { return c ^ ((row >> 1) & 7); }
typedef __attribute__((address_space(3))) void* lds_ptr;
}  // namespace fdma

// Exact float value of byte sel of w as an E4M3 code (gfx950's converter
// decodes the OCP E4M3 format; sel is a constant after unrolling).
__device__ inline float e4m3_byte_f32(uint32_t w, int sel) {
  switch (sel) {
    case 0: return __builtin_amdgcn_cvt_f32_fp8((int)w, 0);
    case 1: return __builtin_amdgcn_cvt_f32_fp8((int)w, 1);
    case 2: return __builtin_amdgcn_cvt_f32_fp8((int)w, 2);
    default: return __builtin_amdgcn_cvt_f32_fp8((int)w, 3);
  }
}

// The mantissa 1.m of a scale (1 for 0) as two equal f16 halves: its three
// fraction bits move from the float32 to the f16 fraction field.
__device__ inline f16x2 mant_f16x2(float scf) {
  const uint32_t h = 0x3C00u | ((__float_as_uint(scf) >> 13) & 0x3FFu);
  return __builtin_bit_cast(f16x2, h * 0x10001u);
}

// 8 exact f16 values of one k step: code dword (8 E2M1 codes), the E4M3
// scale as float (its power of two applies in the convert) and its mantissa.
__device__ inline f16x8 dequant8_f16(uint32_t codes, float scf, f16x2 m2) {
  f16x2 h0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, scf, 0);
  f16x2 h1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, scf, 1);
  f16x2 h2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, scf, 2);
  f16x2 h3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, scf, 3);
  h0 = h0 * m2;
  h1 = h1 * m2;
  h2 = h2 * m2;
  h3 = h3 * m2;
  return f16x8{h0[0], h0[1], h1[0], h1[1], h2[0], h2[1], h3[0], h3[1]};
}

// One 256-element K slab of a wave's MI x NJ fragments from the LDS layout
// above (codes [rows][128 bytes], chunks swizzled; scales [rows][16 bytes]):
// 4 groups of 4 k steps; per group each fragment's 16 code bytes (one b128
// read) and, per pair of steps, its scale.
template <int MI, int NJ>
__device__ __forceinline__ void fp4_slab_mfma(f32x16 (&acc)[MI][NJ], const uint8_t* la, const uint8_t* lb,
                                              const uint8_t* sa, const uint8_t* sb, int wm, int wn, int g, int li) {
  using namespace fdma;
  u32x2 sca[MI], scb[NJ];  // the lane's 8 scale bytes per fragment
#pragma unroll
  for (int i = 0; i < MI; ++i) sca[i] = *reinterpret_cast<const u32x2*>(sa + (wm + i * 32 + li) * 16 + 8 * g);
#pragma unroll
  for (int j = 0; j < NJ; ++j) scb[j] = *reinterpret_cast<const u32x2*>(sb + (wn + j * 32 + li) * 16 + 8 * g);
#pragma unroll
  for (int grp = 0; grp < 4; ++grp) {
    u32x4 ca[MI], cb[NJ];
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const int r = wm + i * 32 + li;
      ca[i] = *reinterpret_cast<const u32x4*>(la + r * RB + 16 * swz(r, 4 * g + grp));
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int r = wn + j * 32 + li;
      cb[j] = *reinterpret_cast<const u32x4*>(lb + r * RB + 16 * swz(r, 4 * g + grp));
    }
#pragma unroll
    for (int hp = 0; hp < 2; ++hp) {  // pairs of k steps share a 16-element scale block
      float sfa[MI], sfb[NJ];
      f16x2 ma[MI], mb[NJ];
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        sfa[i] = e4m3_byte_f32(sca[i][grp >> 1], (grp & 1) * 2 + hp);
        ma[i] = mant_f16x2(sfa[i]);
      }
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        sfb[j] = e4m3_byte_f32(scb[j][grp >> 1], (grp & 1) * 2 + hp);
        mb[j] = mant_f16x2(sfb[j]);
      }
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const int kq = hp * 2 + st;  // step within the group: code dword kq
        f16x8 av[MI], bv[NJ];
#pragma unroll
        for (int i = 0; i < MI; ++i) av[i] = dequant8_f16(ca[i][kq], sfa[i], ma[i]);
#pragma unroll
        for (int j = 0; j < NJ; ++j) bv[j] = dequant8_f16(cb[j][kq], sfb[j], mb[j]);
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
          for (int j = 0; j < NJ; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[i], bv[j], acc[i][j], 0, 0, 0);
      }
    }
  }
}

// The same slab as a software pipeline over its 16 k steps: the fragments of
// step s + 1 are dequantised (and the next group's code words read) while
// step s's MFMAs run, so the matrix unit need not idle behind the conversions
// of its own wave when no other wave of the SIMD computes.
template <int MI, int NJ, int MA = MI>  // MA: the first MA of the MI row fragments are computed
__device__ __forceinline__ void fp4_slab_mfma_pipe(f32x16 (&acc)[MI][NJ], const uint8_t* la, const uint8_t* lb,
                                                   const uint8_t* sa, const uint8_t* sb, int wm, int wn, int g,
                                                   int li) {
  using namespace fdma;
  u32x2 sca[MI], scb[NJ];
#pragma unroll
  for (int i = 0; i < MA; ++i) sca[i] = *reinterpret_cast<const u32x2*>(sa + (wm + i * 32 + li) * 16 + 8 * g);
#pragma unroll
  for (int j = 0; j < NJ; ++j) scb[j] = *reinterpret_cast<const u32x2*>(sb + (wn + j * 32 + li) * 16 + 8 * g);
  u32x4 ca[2][MI], cb[2][NJ];
  f16x8 av[2][MI], bv[2][NJ];
  float sfa[MI], sfb[NJ];
  f16x2 ma[MI], mb[NJ];
  auto read_codes = [&](int grp) {
#pragma unroll
    for (int i = 0; i < MA; ++i) {
      const int r = wm + i * 32 + li;
      ca[grp & 1][i] = *reinterpret_cast<const u32x4*>(la + r * RB + 16 * swz(r, 4 * g + grp));
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int r = wn + j * 32 + li;
      cb[grp & 1][j] = *reinterpret_cast<const u32x4*>(lb + r * RB + 16 * swz(r, 4 * g + grp));
    }
  };
  auto scales = [&](int grp, int hp) {  // step pair hp of group grp shares a 16-element block
#pragma unroll
    for (int i = 0; i < MA; ++i) {
      sfa[i] = e4m3_byte_f32(sca[i][grp >> 1], (grp & 1) * 2 + hp);
      ma[i] = mant_f16x2(sfa[i]);
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      sfb[j] = e4m3_byte_f32(scb[j][grp >> 1], (grp & 1) * 2 + hp);
      mb[j] = mant_f16x2(sfb[j]);
    }
  };
  auto dequant = [&](int st) {  // step st = 4 grp + kq of the slab
    const int grp = st >> 2, kq = st & 3;
#pragma unroll
    for (int i = 0; i < MA; ++i) av[st & 1][i] = dequant8_f16(ca[grp & 1][i][kq], sfa[i], ma[i]);
#pragma unroll
    for (int j = 0; j < NJ; ++j) bv[st & 1][j] = dequant8_f16(cb[grp & 1][j][kq], sfb[j], mb[j]);
  };
  read_codes(0);
  scales(0, 0);
  dequant(0);
#pragma unroll
  for (int st = 0; st < 16; ++st) {
    if (st % 4 == 0 && st + 4 < 16) read_codes((st >> 2) + 1);
    if (st + 1 < 16) {
      if ((st + 1) % 2 == 0) scales((st + 1) >> 2, ((st + 1) >> 1) & 1);
      dequant(st + 1);
    }
#pragma unroll
    for (int i = 0; i < MA; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[st & 1][i], bv[st & 1][j], acc[i][j], 0, 0, 0);
  }
}

template <bool OUT_BF16, int BM, int BN, bool PIPE>
__device__ __forceinline__ void gemm_fwd_dma_body(const uint8_t* __restrict__ a_codes,
                                                             const uint8_t* __restrict__ a_sf,
                                                             const float* __restrict__ a_ts, int a_ts_per_group,
                                                             const uint8_t* __restrict__ b_codes,
                                                             const uint8_t* __restrict__ b_sf,
                                                             const float* __restrict__ b_ts,
                                                             const int32_t* __restrict__ off, int E, int64_t M_total,
                                                             int64_t N, int64_t K, int64_t n_ntiles, int64_t n_all,
                                                             void* __restrict__ c) {
  using namespace fdma;
  constexpr int WM = BM / 2, WN = BN / 2, MI = WM / 32, NJ = WN / 32;
  constexpr int QA = BM / 32, QB = BN / 32;   // 1 KB code loads per wave and slab
  constexpr int SA = BM / 64, SB = BN / 64;   // 64-row scale loads per slab (dealt to the waves)
  __shared__ __attribute__((aligned(16))) uint8_t la0[BM * RB];
  __shared__ __attribute__((aligned(16))) uint8_t lb0[BN * RB];
  __shared__ __attribute__((aligned(16))) uint8_t la1[BM * RB];
  __shared__ __attribute__((aligned(16))) uint8_t lb1[BN * RB];
  __shared__ __attribute__((aligned(16))) uint8_t sa0[BM * 16];
  __shared__ __attribute__((aligned(16))) uint8_t sb0[BN * 16];
  __shared__ __attribute__((aligned(16))) uint8_t sa1[BM * 16];
  __shared__ __attribute__((aligned(16))) uint8_t sb1[BN * 16];
  const int64_t tile = xcd_tile(blockIdx.x, n_all);
  if (tile >= n_all) return;
  const int64_t nt = tile % n_ntiles;
  int e;
  int64_t mt;
  if (!find_m_tile(off, E, BM, tile / n_ntiles, e, mt)) return;
  const int64_t row0 = (int64_t)off[e] + mt * BM;
  const int64_t row_end = (int64_t)off[e + 1] < M_total ? (int64_t)off[e + 1] : M_total;
  const int64_t n0 = nt * BN;
  const int tid = threadIdx.x, l = tid & 63, g = (l >> 5) & 1, li = l & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = (w >> 1) * WM, wn = (w & 1) * WN;
  const int64_t KB = K / 2, KS = K / 16;  // code and scale bytes per row
  const __amdgpu_buffer_rsrc_t rac = make_rsrc(a_codes, (uint64_t)M_total * KB);
  const __amdgpu_buffer_rsrc_t ras = make_rsrc(a_sf, (uint64_t)M_total * KS);
  const __amdgpu_buffer_rsrc_t rbc = make_rsrc(b_codes + (int64_t)e * N * KB, (uint64_t)N * KB);
  const __amdgpu_buffer_rsrc_t rbs = make_rsrc(b_sf + (int64_t)e * N * KS, (uint64_t)N * KS);
  // Rows past the operands are clamped to the last row (valid memory; their
  // results are never stored), so every load is in range.
  uint32_t aoff[QA], boff[QB];
#pragma unroll
  for (int q = 0; q < QA; ++q) {
    const int row = (4 * q + w) * 8 + (l >> 3);
    const int64_t ra = row0 + row < M_total ? row0 + row : M_total - 1;
    aoff[q] = (uint32_t)(ra * KB + 16 * swz(row, l & 7));
  }
#pragma unroll
  for (int q = 0; q < QB; ++q) {
    const int row = (4 * q + w) * 8 + (l >> 3);
    const int64_t rb = n0 + row < N ? n0 + row : N - 1;
    boff[q] = (uint32_t)(rb * KB + 16 * swz(row, l & 7));
  }
  // scale loads: 64 rows (16 bytes each) per instruction; instruction t of
  // the SA + SB is issued by wave t % 4
  uint32_t soff[(SA + SB + 3) / 4];
#pragma unroll
  for (int k = 0; k < (SA + SB + 3) / 4; ++k) {
    const int t = 4 * k + w;
    int64_t r = 0;
    if (t < SA) r = row0 + t * 64 + l < M_total ? row0 + t * 64 + l : M_total - 1;
    else if (t < SA + SB) r = n0 + (t - SA) * 64 + l < N ? n0 + (t - SA) * 64 + l : N - 1;
    soff[k] = (uint32_t)(r * KS);
  }
  auto issue = [&](uint8_t* la, uint8_t* lb, uint8_t* sa, uint8_t* sb, uint32_t ke0) {
    const uint32_t kb = ke0 / 2;
#pragma unroll
    for (int q = 0; q < QA; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rac, (lds_ptr)(la + (4 * q + w) * 1024), 16, aoff[q] + kb, 0, 0, 0);
#pragma unroll
    for (int q = 0; q < QB; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rbc, (lds_ptr)(lb + (4 * q + w) * 1024), 16, boff[q] + kb, 0, 0, 0);
#pragma unroll
    for (int k = 0; k < (SA + SB + 3) / 4; ++k) {
      const int t = 4 * k + w;  // wave-uniform
      if (t < SA)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ras, (lds_ptr)(sa + t * 1024), 16, soff[k] + ke0 / 16, 0, 0, 0);
      else if (t < SA + SB)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rbs, (lds_ptr)(sb + (t - SA) * 1024), 16, soff[k] + ke0 / 16, 0, 0, 0);
    }
  };
  f32x16 acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = f32x16{};
  auto compute = [&](const uint8_t* la, const uint8_t* lb, const uint8_t* sa, const uint8_t* sb) {
    fp4_slab_mfma<MI, NJ>(acc, la, lb, sa, sb, wm, wn, g, li);
  };
  auto compute_pipe = [&](const uint8_t* la, const uint8_t* lb, const uint8_t* sa, const uint8_t* sb) {
    fp4_slab_mfma_pipe<MI, NJ>(acc, la, lb, sa, sb, wm, wn, g, li);
  };
  // waves whose rows all lie past a small expert's last row skip their MFMAs
  const int64_t left = row_end - (row0 + wm);
  const int active = __builtin_amdgcn_readfirstlane(left > 0 ? 1 : 0);
  auto sync = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0);  // vmcnt(0) expcnt(0) lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };
  auto slab = [&](const uint8_t* la, const uint8_t* lb, const uint8_t* sa, const uint8_t* sb) {
    if (PIPE) compute_pipe(la, lb, sa, sb);
    else compute(la, lb, sa, sb);
  };
  const uint32_t nk = (uint32_t)(K / BKE);
  issue(la0, lb0, sa0, sb0, 0);
  uint32_t s = 0;
  for (; s + 2 <= nk; s += 2) {
    sync();
    issue(la1, lb1, sa1, sb1, (s + 1) * BKE);
    if (active) slab(la0, lb0, sa0, sb0);
    sync();
    if (s + 2 < nk) issue(la0, lb0, sa0, sb0, (s + 2) * BKE);
    if (active) slab(la1, lb1, sa1, sb1);
  }
  if (s < nk) {
    sync();
    if (active) slab(la0, lb0, sa0, sb0);
  }
  // Epilogue: 32-row bands of each wave's tile through LDS (free after the
  // last barrier), scaled by S_a * S_b, written as row-contiguous 16-byte
  // (f32) or 8-byte (bf16) stores.
  sync();
  const float sab = a_ts[a_ts_per_group ? e : 0] * b_ts[e];
  constexpr int BS = WN + 4;
  // each wave's 32-row float band in its own freed code buffer
  float* band = reinterpret_cast<float*>(w == 0 ? la0 : (w == 1 ? lb0 : (w == 2 ? la1 : lb1)));
  static_assert(32 * BS * 4 <= (BM < BN ? BM : BN) * RB, "epilogue band does not fit a code buffer");
#pragma unroll
  for (int i = 0; i < MI; ++i) {
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) band[((v >> 2) * 8 + g * 4 + (v & 3)) * BS + j * 32 + li] = acc[i][j][v] * sab;
    __builtin_amdgcn_wave_barrier();
    constexpr int QPR = WN / 4;  // column quads per band row
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

// One kernel per configuration (the body is a device template).
#define MOE4_FWD_DMA_KERNEL(NAME, OUT_BF16, BM, BN, MINB, PIPE)                                                         \
  __global__ void __launch_bounds__(fdma::NT, MINB)                                                               \
      NAME(const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_sf, const float* __restrict__ a_ts,  \
           int a_ts_per_group, const uint8_t* __restrict__ b_codes, const uint8_t* __restrict__ b_sf,             \
           const float* __restrict__ b_ts, const int32_t* __restrict__ off, int E, int64_t M_total, int64_t N,    \
           int64_t K, int64_t n_ntiles, int64_t n_all, void* __restrict__ c) {                                    \
    gemm_fwd_dma_body<OUT_BF16, BM, BN, PIPE>(a_codes, a_sf, a_ts, a_ts_per_group, b_codes, b_sf, b_ts, off, E, M_total, \
                                        N, K, n_ntiles, n_all, c);                                                 \
  }
MOE4_FWD_DMA_KERNEL(k_gemm_fwd_dma_bf16_128, true, 128, 128, 2, false)
MOE4_FWD_DMA_KERNEL(k_gemm_fwd_dma_f32_128, false, 128, 128, 2, false)
#undef MOE4_FWD_DMA_KERNEL

// ------------------------------------------- warp-specialised persistent variant
// K % 256 == 0.  One workgroup of 8 waves per CU walks 128 x 128 tiles.
// Four producer waves only issue direct-to-LDS loads of 256-element K slabs
// (the layout of the kernel above: 16 KB of codes and 2 KB of scales per
// operand) into a four-stage ring; four consumer waves only read LDS,
// dequantise and run the f16 MFMAs (64 x 64 each) and store their results
// straight from the accumulators.  gfx950 counts a wave's loads and stores on
// one counter that completes in issue order, so a wave that both loads and
// stores would wait for its stores' acknowledgements before each slab; here
// no wave does both.  One barrier per slab: producers wait for slab s with an
// explicit count (the later slabs stay in flight), consumers only for their
// own LDS reads of slab s - 1.  Tiles: m-tiles in expert order, dealt to the
// XCDs in rectangles of one band of m-tiles at a time (DgSplit), so that an
// XCD's concurrent tiles share A rows and B rows in its L2 and all XCDs read
// the same experts' weights at about the same time.
namespace fws {
constexpr int TM = 128;
// TN = 128: four stages, four consumer waves; TN = 256: two 54 KB stages (all
// the LDS allows) and eight consumer waves, so that two of a SIMD's three
// waves compute and one's conversions overlap the other's MFMAs.  Consumers
// own 64 x 64 blocks either way.
template <int TN>
struct Cfg {
  static constexpr int NCW = TN / 32, NT = 64 * (NCW + 4);
  static constexpr int CODE_A = TM * fdma::RB, CODE_B = TN * fdma::RB;  // per stage
  static constexpr int SCL_A = TM * 16, SCL_B = TN * 16;
  static constexpr int STAGE = CODE_A + CODE_B + SCL_A + SCL_B;
  static constexpr int S = TN == 128 ? 4 : 2;
  static constexpr int QB = TN / 32;            // B code row groups per producer wave
  static constexpr int NS = TN == 128 ? 1 : 2;  // scale groups per producer wave
  static constexpr int I = 4 + QB + NS;         // loads per producer wave and slab
};
constexpr int wait_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
constexpr int WAIT_LGKM0 = 15 | (3 << 14) | (7 << 4);
}  // namespace fws

// quad_perm [1,0,3,2] and [2,3,0,1]: the value of lane l ^ 1 and of lane l ^ 2
__device__ inline float dpp_xor1(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
}
__device__ inline float dpp_xor2(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));
}

// The combine-path payload of 16 rows x 32 columns of one 32 x 32 output
// fragment (values in the wave's LDS block hb [16 rows][36 floats]): lane l
// takes row l / 4, columns 8 (l % 4) .. + 7 of the block, so the transform's
// distance-1, 2, 4 stages stay in the lane and the distance-8 and 16 stages
// (and the block maximum) pair lanes l ^ 1 and l ^ 2.  Writes the lane's 8
// int8 codes at row r0 + l / 4, column c0 + 8 (l % 4) of the payload and,
// from lanes l % 4 == 0, the block's E8M0 byte.
__device__ inline void hmx8_half(const float* hb, int l, __amdgpu_buffer_rsrc_t rH, __amdgpu_buffer_rsrc_t rS,
                                 uint32_t r0, uint32_t c0, uint32_t N) {
  const int r = l >> 2, q = l & 3;
  const f32x4 lo = *reinterpret_cast<const f32x4*>(hb + r * 36 + 8 * q);
  const f32x4 hi = *reinterpret_cast<const f32x4*>(hb + r * 36 + 8 * q + 4);
  float v[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
  for (int h = 1; h < 8; h <<= 1)
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (!(i & h)) {
        const float a = v[i], b = v[i + h];
        v[i] = a + b;
        v[i + h] = a - b;
      }
  // distance 8 and 16: the partner is lane l ^ 1, then l ^ 2; the lower lane
  // keeps a + b, the upper one a - b with a the lower lane's value
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float o = dpp_xor1(v[i]);
    v[i] = (q & 1) ? o - v[i] : v[i] + o;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float o = dpp_xor2(v[i]);
    v[i] = (q & 2) ? o - v[i] : v[i] + o;
  }
  float am = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) am = fmaxf(am, fabsf(v[i]));
  am = fmaxf(am, dpp_xor1(am));
  am = fmaxf(am, dpp_xor2(am));
  int ex = -127;
  if (am > 0.0f) {
    ex = __builtin_amdgcn_frexp_expf(am) - 1;
    ex = ex < -127 ? -127 : ex;
  }
  uint32_t w0 = 0u, w1 = 0u;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float c = __builtin_rintf(__builtin_amdgcn_ldexpf(v[i], 6 - ex));
    c = fminf(fmaxf(c, -127.0f), 127.0f);
    const uint32_t b = ((uint32_t)(int)c & 0xFFu) << (8 * (i & 3));
    if (i < 4) w0 |= b; else w1 |= b;
  }
  const uint32_t row = r0 + (uint32_t)r;
  __builtin_amdgcn_raw_buffer_store_b64(u32x2{w0, w1}, rH, row * N + c0 + 8u * (uint32_t)q, 0, 0);
  if (q == 0) __builtin_amdgcn_raw_buffer_store_b8((unsigned char)(ex + 127), rS, row * (N / 32) + c0 / 32, 0, 0);
}

// HMX8 (float32 output only): the epilogue also writes the combine-path
// payload of the stored values: per row and 32-column block, the Sylvester
// H_32 transform as five butterfly stages (partner distance 1, 2, 4, 8, 16;
// the lower position keeps a + b, the upper a - b), the block's E8M0 exponent
// floor(log2 max|y|) (-127 for zeros) and int8 codes rne(y 2^(6 - e))
// clamped to +-127: the steps and float32 roundings of moe_hmx8_quant, byte
// for byte.  A fragment's lane holds one column of each row; each half of the
// fragment goes through a 2.3 KB LDS block of the wave to the quantiser's
// layout (8 consecutive columns per lane: hmx8_half).
template <bool OUT_BF16, int TN, bool HMX8 = false>
__global__ void __launch_bounds__(fws::Cfg<TN>::NT, 1)
    k_gemm_fwd_ws(const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_sf, const float* __restrict__ a_ts,
                  int a_ts_per_group, const uint8_t* __restrict__ b_codes, const uint8_t* __restrict__ b_sf,
                  const float* __restrict__ b_ts, const int32_t* __restrict__ off, int E, int64_t M_total, int64_t N,
                  int64_t K, DgSplit sp, void* __restrict__ c, uint32_t* __restrict__ silu_amax,
                  const float* __restrict__ act_tab, int8_t* __restrict__ hcodes = nullptr,
                  uint8_t* __restrict__ hsf = nullptr) {
  static_assert(!HMX8 || !OUT_BF16, "the combine-path payload is made from the float32 output");
  using namespace fws;
  using fdma::lds_ptr;
  using fdma::swz;
  using C = Cfg<TN>;
  constexpr int S = C::S, STAGE = C::STAGE, I = C::I, NCW = C::NCW;
  __shared__ __attribute__((aligned(16))) uint8_t ring[S * STAGE];
  __shared__ uint32_t s_nmt;
  __shared__ __attribute__((aligned(16))) float hbuf[HMX8 ? NCW * 16 * 36 : 4];  // (HMX8) a block per consumer wave
  const int tid = threadIdx.x, l = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  // total m-tiles (before any load into LDS is in flight)
  if (w == 0) {
    uint32_t n = 0;
    for (int e = l; e < E; e += 64) n += (uint32_t)((off[e + 1] - off[e] + TM - 1) / TM);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) n += __shfl_xor(n, o, 64);
    if (l == 0) s_nmt = n;
  }
  __syncthreads();
  const uint32_t n_nt = (uint32_t)(N / TN), n_mt = s_nmt;  // N % TN == 0 (checked at launch)
  const uint32_t KB = (uint32_t)(K / 2), KS = (uint32_t)(K / 16), nk = (uint32_t)(K / fdma::BKE);
  // this workgroup's tiles: q = q0, q0 + stride, ... of its XCD (see DgSplit)
  const uint32_t xcd = blockIdx.x % 8, stride = (gridDim.x - xcd + 7) / 8, q0 = blockIdx.x / 8;
  const uint32_t sm = (8 / sp.xb) * sp.pm, q_end = (n_mt + sm - 1) / sm * (sp.pm * sp.pn);

  if (w >= NCW) {
    // ---- producer pw: rows 32 pw .. 32 pw + 31 of A's codes, TN / 4 rows of
    // B's, and 64-row scale groups: TN = 128: A 0-63, A 64-127, B 0-63,
    // B 64-127; TN = 256: A 0-63 + B 0-63, A 64-127 + B 64-127, B 128-191 +
    // A 0-63, B 192-255 + A 64-127 (two waves load an A group twice, so that
    // every producer issues the same number of loads: the waits count them)
    const int pw = w - NCW;
    const __amdgpu_buffer_rsrc_t rac = make_rsrc(a_codes, (uint64_t)M_total * KB);
    const __amdgpu_buffer_rsrc_t ras = make_rsrc(a_sf, (uint64_t)M_total * KS);
    __amdgpu_buffer_rsrc_t rbc = rac, rbs = ras;
    // (fixed sizes: the first C::QB and C::NS are used; hipcc's host pass rejects
    // arrays sized by the template argument inside the lambdas)
    uint32_t aoff[4], boff[8], soff[2];
    auto sgrp = [&](int k, bool& opb, int& r0) {  // scale group k: operand B?, first row
      if (TN == 128) {
        opb = pw >= 2;
        r0 = 64 * (pw & 1);
      } else {  // waves 0, 1: A then B; waves 2, 3: B then A
        opb = pw < 2 ? k == 1 : k == 0;
        r0 = opb ? 64 * pw : 64 * (pw & 1);
      }
    };
    MtCursor<TM> cur;
    uint32_t pt = q0, ps = 0;
    bool more = false;
    auto seek = [&]() {
      uint32_t mi = 0, nt = 0;
      while (pt < q_end && !sp.tile(xcd, pt, n_mt, n_nt, mi, nt)) pt += stride;
      more = pt < q_end && cur.seek(off, E, mi);
      if (!more) return;
      const int e = cur.e;
      const uint32_t mt = mi - cur.first;
      const int64_t row0 = (int64_t)ld_const(off, e) + (int64_t)mt * TM, n0 = (int64_t)nt * TN;
      rbc = make_rsrc(b_codes + (int64_t)e * N * KB, (uint64_t)N * KB);
      rbs = make_rsrc(b_sf + (int64_t)e * N * KS, (uint64_t)N * KS);
      // rows past the operands are clamped to the last row: valid memory whose
      // results are never stored
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = 32 * pw + 8 * q + (l >> 3);
        const int64_t ra = row0 + r < M_total ? row0 + r : M_total - 1;
        aoff[q] = (uint32_t)ra * KB + 16u * (uint32_t)swz(r, l & 7);
      }
#pragma unroll
      for (int q = 0; q < C::QB; ++q) {
        const int r = (TN / 4) * pw + 8 * q + (l >> 3);
        const int64_t rb = n0 + r < N ? n0 + r : N - 1;
        boff[q] = (uint32_t)rb * KB + 16u * (uint32_t)swz(r, l & 7);
      }
#pragma unroll
      for (int k = 0; k < C::NS; ++k) {
        bool opb;
        int r0;
        sgrp(k, opb, r0);
        const int sr = r0 + l;
        const int64_t srow = opb ? (n0 + sr < N ? n0 + sr : N - 1) : (row0 + sr < M_total ? row0 + sr : M_total - 1);
        soff[k] = (uint32_t)srow * KS;
      }
      ps = 0;
    };
    seek();
    auto issue = [&](int st) {
      uint8_t* base = ring + st * STAGE;
      const uint32_t kb = ps * (uint32_t)fdma::RB, ksb = ps * 16u;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rac, (lds_ptr)(base + (4 * pw + q) * 1024), 16, aoff[q] + kb, 0, 0, 0);
#pragma unroll
      for (int q = 0; q < C::QB; ++q)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rbc, (lds_ptr)(base + C::CODE_A + (C::QB * pw + q) * 1024), 16,
                                                 boff[q] + kb, 0, 0, 0);
#pragma unroll
      for (int k = 0; k < C::NS; ++k) {
        bool opb;
        int r0;
        sgrp(k, opb, r0);
        uint8_t* sb = base + C::CODE_A + C::CODE_B + (opb ? C::SCL_A : 0) + r0 * 16;
        if (opb) __builtin_amdgcn_raw_ptr_buffer_load_lds(rbs, (lds_ptr)sb, 16, soff[k] + ksb, 0, 0, 0);
        else __builtin_amdgcn_raw_ptr_buffer_load_lds(ras, (lds_ptr)sb, 16, soff[k] + ksb, 0, 0, 0);
      }
      if (++ps == nk) {
        pt += stride;
        seek();
      }
    };
    uint32_t n_iss = 0;
    for (int st = 0; st < S - 1 && more; ++st) {
      issue(st);
      ++n_iss;
    }
    for (uint32_t gs = 0; gs < n_iss; ++gs) {
      // slab gs landed (later slabs may still be in flight), then the barrier
      const uint32_t rem = n_iss - 1 - gs;
      __builtin_amdgcn_sched_barrier(0);
      if (rem >= 2) __builtin_amdgcn_s_waitcnt(wait_vm(2 * I));
      else if (rem == 1) __builtin_amdgcn_s_waitcnt(wait_vm(I));
      else __builtin_amdgcn_s_waitcnt(wait_vm(0));
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("" ::: "memory");
      if (more) {
        issue((int)((gs + S - 1) % S));
        ++n_iss;
      }
    }
    return;
  }
  // ---- consumers: wave w owns the 64 x 64 block (w / (TN / 64), w % (TN / 64))
  constexpr int MI = 2, NJ = 2;
  const int g = (l >> 5) & 1, li = l & 31;
  const int wm = (w / (TN / 64)) * 64, wn = (w % (TN / 64)) * 64;
  f32x16 acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = f32x16{};
  constexpr int ESZ = OUT_BF16 ? 2 : 4;
  const uint32_t ld = (uint32_t)N * ESZ;  // output row pitch in bytes
  const uint32_t lane_off = (uint32_t)(g * 4) * ld + (uint32_t)li * ESZ;
  float* hb = hbuf + (HMX8 ? w * 16 * 36 : 0);  // (HMX8) this consumer wave's block
  MtCursor<TM> cur;
  uint32_t gs = 0;
  for (uint32_t q = q0; q < q_end; q += stride) {
    uint32_t mi, nt;
    if (!sp.tile(xcd, q, n_mt, n_nt, mi, nt)) continue;
    if (!cur.seek(off, E, mi)) break;
    const int e = cur.e;
    const uint32_t mt = mi - cur.first;
    const int64_t row0 = (int64_t)ld_const(off, e) + (int64_t)mt * TM, n0 = (int64_t)nt * TN;
    const int64_t row_end = (int64_t)ld_const(off, e + 1) < M_total ? (int64_t)ld_const(off, e + 1) : M_total;
    // waves whose rows all lie past the expert's last row skip their MFMAs,
    // and those with only their first 32 rows in it compute those alone (the
    // other accumulators stay zero and their stores fall past the descriptor)
    const bool active = row0 + wm < row_end, active2 = row0 + wm + 32 < row_end;
    for (uint32_t s = 0; s < nk; ++s, ++gs) {
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(WAIT_LGKM0);
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("" ::: "memory");
      const uint8_t* base = ring + (gs % S) * STAGE;
      const uint8_t* sa = base + C::CODE_A + C::CODE_B;
      if (active2) fp4_slab_mfma_pipe<MI, NJ>(acc, base, base + C::CODE_A, sa, sa + C::SCL_A, wm, wn, g, li);
      else if (active) fp4_slab_mfma_pipe<MI, NJ, 1>(acc, base, base + C::CODE_A, sa, sa + C::SCL_A, wm, wn, g, li);
    }
    // epilogue: S_a * S_b, then each value straight from the accumulators;
    // the descriptor covers the tile's rows up to the expert's last, so
    // stores of rows past it are dropped
    const float sab = __int_as_float(ld_const(reinterpret_cast<const int32_t*>(a_ts), a_ts_per_group ? e : 0)) *
                      __int_as_float(ld_const(reinterpret_cast<const int32_t*>(b_ts), e));
    const int64_t nrows = row_end - row0 < TM ? row_end - row0 : TM;
    const __amdgpu_buffer_rsrc_t rC = make_rsrc(static_cast<uint8_t*>(c) + row0 * (int64_t)ld, (uint64_t)nrows * ld);
    // With silu_amax (bf16 U): the expert's max |silu(u)| over the stored
    // values of its rows, from three extremes of the bf16 patterns (silu is
    // non-decreasing on [0, inf); |silu| is monotone on each side of its
    // minimum, split by the adjacent bf16 values -1.28125 and -1.2734375),
    // then one atomic maximum per wave and tile.
    constexpr uint32_t M1 = 0x3FA4u;  // |-1.28125| in bf16
    const bool amx = OUT_BF16 && silu_amax != nullptr && active;
    // (HMX8) the payload's codes and scale bytes of the tile's rows
    const __amdgpu_buffer_rsrc_t rH = make_rsrc(HMX8 ? hcodes + row0 * N : nullptr, HMX8 ? (uint64_t)nrows * N : 0);
    const __amdgpu_buffer_rsrc_t rS =
        make_rsrc(HMX8 ? hsf + row0 * (N / 32) : nullptr, HMX8 ? (uint64_t)nrows * (N / 32) : 0);
    uint32_t pmax = 0u, nlo = 0x8000u, nhi = 0u;
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        if (active) {
          const uint32_t fo = (uint32_t)(wm + i * 32) * ld + (uint32_t)(n0 + wn + j * 32) * ESZ;
          const int rows_left = (int)nrows - (wm + i * 32 + g * 4);
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const uint32_t so = fo + (uint32_t)((v >> 2) * 8 + (v & 3)) * ld;
            const float x = acc[i][j][v] * sab;
            if (OUT_BF16) {
              const uint32_t b = f32_to_bf16_bits(x);
              __builtin_amdgcn_raw_buffer_store_b16((unsigned short)b, rC, lane_off, so, 2);
              if (amx && (v >> 2) * 8 + (v & 3) < rows_left) {  // the stored values of the expert's rows
                const uint32_t m = b & 0x7FFFu;
                const bool neg = b >= 0x8000u;
                pmax = max(pmax, neg ? 0u : m);
                nlo = min(nlo, neg && m >= M1 ? m : 0x8000u);
                nhi = max(nhi, neg && m < M1 ? m : 0u);
              }
            } else {
              __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), rC, lane_off, so, 2);
            }
            if constexpr (HMX8) {  // row (v / 4) 8 + 4 g + v % 4 of the fragment, column li
              hb[((v & 7) >> 2) * 8 * 36 + (g * 4 + (v & 3)) * 36 + li] = x;
              if ((v & 7) == 7) {  // a 16-row half is in the block
                asm volatile("" ::: "memory");
                hmx8_half(hb, l, rH, rS, (uint32_t)(wm + i * 32 + (v >> 3) * 16), (uint32_t)(n0 + wn + j * 32),
                          (uint32_t)N);
                asm volatile("" ::: "memory");
              }
            }
          }
        }
      }
    if (amx) {  // the wave's extremes (folded in the store loop above), then one atomic
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) {
        pmax = max(pmax, (uint32_t)__shfl_xor((int)pmax, o, 64));
        nlo = min(nlo, (uint32_t)__shfl_xor((int)nlo, o, 64));
        nhi = max(nhi, (uint32_t)__shfl_xor((int)nhi, o, 64));
      }
      if (l == 0) {
        float t = act_eval<false>(pmax, act_tab);
        if (nlo < 0x8000u) t = fmaxf(t, fabsf(act_eval<false>(0x8000u | nlo, act_tab)));
        t = fmaxf(t, fabsf(act_eval<false>(0x8000u | nhi, act_tab)));
        atomicMax(silu_amax + e, __float_as_uint(t));  // t >= 0: bit order = value order
      }
    }
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
  }
}

// ------------------------------------------------ few rows per expert
// When the experts hold a few rows each (a rollout batch: about 10 of 512
// tokens' 8 slots per expert), the forward is bound by streaming the NVFP4
// weights once, and a 128-row M tile would compute mostly padding.  Here the
// weight rows take the MFMA's M side and the expert's tokens its N side, 16
// at a time (v_mfma_f32_16x16x32_f16): workgroup (weight-row block, expert),
// four waves of 32 weight rows (two 16-row MFMA blocks) each, all of the
// expert's tokens in passes of 16 (an expert of 17 to 32 rows streams its
// weights twice).  No LDS: every lane
// loads, per K step of 256 and weight row, 32 code bytes (64 values) and the
// dword of their four E4M3 scales, the next K step in flight; the token codes
// (from L2: every weight-row block of the expert reads them) likewise.  Both
// operands are dequantised exactly to f16 in registers as in the staged
// kernels (FP4 -> f16 by the scale's power of two, times its mantissa).  K
// order inside a step: lane group q = lane / 16 holds values 64 q .. 64 q + 63
// of the step, and MFMA i takes 8 q .. of each group's 8 i .. 8 i + 7: the same
// for both operands, so each MFMA sums 32 matching products.
namespace fsk {
constexpr int NT = 256, WB = 2, WROWS = 16 * WB, KSTEP = 256, TG = 1;   // WB 16-row blocks per wave
}

struct SkOp {          // one row's share of a K step: 64 values
  u32x4 q[2];
  uint32_t s;
};

__device__ inline void sk_load(SkOp& o, const uint8_t* codes, const uint8_t* sf, int64_t row, int64_t K, int64_t k0,
                               int qg) {
  const u32x4* p = reinterpret_cast<const u32x4*>(codes + row * (K / 2) + k0 / 2 + 32 * qg);
  o.q[0] = p[0];
  o.q[1] = p[1];
  o.s = *reinterpret_cast<const uint32_t*>(sf + row * (K / 16) + k0 / 16 + 4 * qg);
}

// The four blocks' scales of a row share: each as the float32 scale (whose
// power of two the converter applies) and its mantissa 1.m in f16.
struct SkScale {
  float scf;
  f16x2 m2;
};

// block blk's scale of a row share
__device__ inline SkScale sk_scale(const SkOp& o, int blk) {
  SkScale sc;
  sc.scf = e4m3_to_f32((o.s >> (8 * blk)) & 0xFFu);
  const _Float16 mh = (_Float16)mant_factor(sc.scf);
  sc.m2 = f16x2{mh, mh};
  return sc;
}

// f16 values 8 i .. 8 i + 7 of the row's 64 (block i / 2 of four, half i % 2)
__device__ inline f16x8 sk_deq8(const SkOp& o, const SkScale& sc, int i) {
  const float scf = sc.scf;
  const f16x2 m2 = sc.m2;
  const uint32_t word = o.q[i >> 2][i & 3];     // 8 values = 4 bytes
  f16x8 r;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    f16x2 h = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4((word >> (8 * b)) & 0xFFu, scf, 0);
    h = h * m2;
    r[2 * b] = h[0];
    r[2 * b + 1] = h[1];
  }
  return r;
}

template <bool OUT_BF16>
__global__ void __launch_bounds__(fsk::NT, 3)
    k_gemm_fwd_skinny(const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_sf,
                      const float* __restrict__ a_ts, int a_ts_per_group, const uint8_t* __restrict__ b_codes,
                      const uint8_t* __restrict__ b_sf, const float* __restrict__ b_ts,
                      const int32_t* __restrict__ off, int E, int64_t M_total, int64_t N, int64_t K,
                      void* __restrict__ c, uint32_t* __restrict__ silu_amax, const float* __restrict__ act_tab) {
  using namespace fsk;
  const int e = blockIdx.y;
  const int l = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t r0 = off[e], r1 = off[e + 1] < M_total ? off[e + 1] : M_total;
  const int64_t n0 = (int64_t)blockIdx.x * ((NT / 64) * WROWS) + (int64_t)wv * WROWS;
  if (r1 <= r0 || n0 >= N) return;                      // no tokens, or no weight rows for this wave
  const int li = l & 15, qg = l >> 4;
  const uint8_t* bc = b_codes + (int64_t)e * N * (K / 2);
  const uint8_t* bs = b_sf + (int64_t)e * N * (K / 16);
  const float sab = a_ts[a_ts_per_group ? e : 0] * b_ts[e];
  const int64_t nks = K / KSTEP;
  const bool amx = OUT_BF16 && silu_amax != nullptr;
  uint32_t pmax = 0u, nlo = 0x8000u, nhi = 0u;
  constexpr uint32_t M1 = 0x3FA4u;  // |-1.28125| in bf16: the SiLU amax split (as k_gemm_fwd_ws)
  for (int64_t p0 = r0; p0 < r1; p0 += 16 * TG) {     // passes of 32 tokens
    f32x4 acc[WB][TG];
#pragma unroll
    for (int b = 0; b < WB; ++b)
#pragma unroll
      for (int t = 0; t < TG; ++t) acc[b][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    int64_t trow[TG];
#pragma unroll
    for (int t = 0; t < TG; ++t) {    // token rows past the expert are clamped (never stored)
      const int64_t r = p0 + 16 * t + li;
      trow[t] = r < r1 ? r : r1 - 1;
    }
    // two register sets, named (not indexed by the step's parity, which would
    // make the compiler select between them and wait for both)
    SkOp wa[WB], xa[TG], wb[WB], xb[TG];
    auto fetch = [&](SkOp (&w)[WB], SkOp (&x)[TG], int64_t k0) {
#pragma unroll
      for (int b = 0; b < WB; ++b) sk_load(w[b], bc, bs, n0 + 16 * b + li, K, k0, qg);
#pragma unroll
      for (int t = 0; t < TG; ++t) sk_load(x[t], a_codes, a_sf, trow[t], K, k0, qg);
    };
    auto compute = [&](const SkOp (&w)[WB], const SkOp (&x)[TG]) {
#pragma unroll
      for (int blk = 0; blk < 4; ++blk) {      // the row share's four 16-value scale blocks
        SkScale ws[WB], xs[TG];
#pragma unroll
        for (int b = 0; b < WB; ++b) ws[b] = sk_scale(w[b], blk);
#pragma unroll
        for (int t = 0; t < TG; ++t) xs[t] = sk_scale(x[t], blk);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int i = 2 * blk + h;
          f16x8 xv[TG];
#pragma unroll
          for (int t = 0; t < TG; ++t) xv[t] = sk_deq8(x[t], xs[t], i);
#pragma unroll
          for (int b = 0; b < WB; ++b) {
            const f16x8 wvv = sk_deq8(w[b], ws[b], i);
#pragma unroll
            for (int t = 0; t < TG; ++t)
              acc[b][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wvv, xv[t], acc[b][t], 0, 0, 0);
          }
        }
      }
    };
    fetch(wa, xa, 0);
    for (int64_t ks = 0; ks < nks; ks += 2) {      // the next step in flight during each step
      if (ks + 1 < nks) fetch(wb, xb, (ks + 1) * KSTEP);
      compute(wa, xa);
      if (ks + 1 >= nks) break;
      if (ks + 2 < nks) fetch(wa, xa, (ks + 2) * KSTEP);
      compute(wb, xb);
    }
    // out[token][n]: lane (li, qg) holds token li of the group and weight rows
    // n0 + 16 b + 4 qg .. + 3: four consecutive output columns
#pragma unroll
    for (int t = 0; t < TG; ++t) {
      const int64_t row = p0 + 16 * t + li;
      if (row >= r1) continue;
#pragma unroll
      for (int b = 0; b < WB; ++b) {
        const int64_t col = n0 + 16 * b + 4 * qg;
        const f32x4 v = acc[b][t] * sab;
        if (OUT_BF16) {
          const uint32_t h0 = f32_to_bf16_bits(v[0]), h1 = f32_to_bf16_bits(v[1]);
          const uint32_t h2 = f32_to_bf16_bits(v[2]), h3 = f32_to_bf16_bits(v[3]);
          *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(c) + row * N + col) = u32x2{h0 | (h1 << 16), h2 | (h3 << 16)};
          if (amx) {
            const uint32_t hb[4] = {h0, h1, h2, h3};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const uint32_t m = hb[q] & 0x7FFFu;
              const bool neg = hb[q] >= 0x8000u;
              pmax = max(pmax, neg ? 0u : m);
              nlo = min(nlo, neg && m >= M1 ? m : 0x8000u);
              nhi = max(nhi, neg && m < M1 ? m : 0u);
            }
          }
        } else {
          *reinterpret_cast<f32x4*>(static_cast<float*>(c) + row * N + col) = v;
        }
      }
    }
  }
  if (amx) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      pmax = max(pmax, (uint32_t)__shfl_xor((int)pmax, o, 64));
      nlo = min(nlo, (uint32_t)__shfl_xor((int)nlo, o, 64));
      nhi = max(nhi, (uint32_t)__shfl_xor((int)nhi, o, 64));
    }
    if (l == 0) {
      float t = act_eval<false>(pmax, act_tab);
      if (nlo < 0x8000u) t = fmaxf(t, fabsf(act_eval<false>(0x8000u | nlo, act_tab)));
      t = fmaxf(t, fabsf(act_eval<false>(0x8000u | nhi, act_tab)));
      atomicMax(silu_amax + e, __float_as_uint(t));
    }
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

template <bool OUT_BF16, int BM, int BN, int MINB>
static void launch_fwd_dma(hipStream_t s, const uint8_t* ac, const uint8_t* as, const float* ats, int apg,
                           const uint8_t* bc, const uint8_t* bs, const float* bts, const int32_t* off, int E, int64_t M,
                           int64_t N, int64_t K, void* c) {
  const int64_t n_nt = (N + BN - 1) / BN;
  const int64_t n_all = n_nt * ((M + BM - 1) / BM + E);
  static_assert(BM == 128 && BN == 128 && MINB == 2, "the direct-to-LDS forward kernel is built for 128x128 tiles");
  const dim3 grid((unsigned)xcd_grid(n_all));
  hipLaunchKernelGGL(OUT_BF16 ? k_gemm_fwd_dma_bf16_128 : k_gemm_fwd_dma_f32_128, grid, dim3(fdma::NT), 0, s, ac, as,
                     ats, apg, bc, bs, bts, off, E, M, N, K, n_nt, n_all, c);
}

// Kernel choice: 11 = warp-specialised persistent 128x256 (K % 256 == 0 and
// N % 256 == 0), 10 = the same with 128x128 tiles (N % 128 == 0), both with
// 32-bit operand offsets and tile indices; else 9 = direct-to-LDS 128x128
// (2 blocks/CU) when K % 256 == 0; else 0 = 128x128 register-staged.
static int cu_count_f() {
  static int n[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (n[dev] == 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
    n[dev] = v;
  }
  return n[dev];
}

// Persistent grid of the warp-specialised forward kernels: one workgroup per
// CU, at least one per XCD (the tile order deals each XCD its own tiles).
static int fws_grid() { return cu_count_f() < 8 ? 8 : cu_count_f(); }

// 12 = the few-rows-per-expert kernel (k_gemm_fwd_skinny): K % 256 == 0,
// N % 64 == 0, at most 32 rows per expert on average.
static int fwd_choice(int64_t M, int64_t N, int64_t K, int E) {
  if (K % fsk::KSTEP == 0 && N % fsk::WROWS == 0 && M <= (int64_t)32 * E && M * (K / 2) < ((int64_t)1 << 40))
    return 12;
  int choice = N % 256 == 0 ? 11 : 10;
  // the persistent kernels' 32-bit operand offsets and tile indices
  if ((choice == 10 || choice == 11) &&
      (N % 128 != 0 || M * (K / 2) >= ((int64_t)1 << 31) || N * (K / 2) >= ((int64_t)1 << 31)))
    choice = 9;
  if (K % fdma::BKE != 0) choice = 0;
  return choice;
}

template <bool OUT_BF16>
static void launch_fwd(hipStream_t s, const uint8_t* ac, const uint8_t* as, const float* ats, int apg,
                       const uint8_t* bc, const uint8_t* bs, const float* bts, const int32_t* off, int E, int64_t M,
                       int64_t N, int64_t K, void* c, uint32_t* silu_amax = nullptr, const float* act_tab = nullptr) {
  const int choice = fwd_choice(M, N, K, E);
  if (choice == 12) {
    const int64_t wg_rows = (fsk::NT / 64) * fsk::WROWS;
    const dim3 grid((unsigned)((N + wg_rows - 1) / wg_rows), (unsigned)E);
    hipLaunchKernelGGL((k_gemm_fwd_skinny<OUT_BF16>), grid, dim3(fsk::NT), 0, s, ac, as, ats, apg, bc, bs, bts, off, E,
                       M, N, K, c, silu_amax, act_tab);
    return;
  }
  if (choice == 10) {
    hipLaunchKernelGGL((k_gemm_fwd_ws<OUT_BF16, 128>), dim3((unsigned)fws_grid()), dim3(fws::Cfg<128>::NT), 0, s, ac, as,
                       ats, apg, bc, bs, bts, off, E, M, N, K, dg_split(N / 128, fws::TM, 128), c, silu_amax, act_tab);
    return;
  }
  if (choice == 11) {
    hipLaunchKernelGGL((k_gemm_fwd_ws<OUT_BF16, 256>), dim3((unsigned)fws_grid()), dim3(fws::Cfg<256>::NT), 0, s, ac, as,
                       ats, apg, bc, bs, bts, off, E, M, N, K, dg_split(N / 256, fws::TM, 256), c, silu_amax, act_tab);
    return;
  }
  if (choice == 9) {
    launch_fwd_dma<OUT_BF16, 128, 128, 2>(s, ac, as, ats, apg, bc, bs, bts, off, E, M, N, K, c);
    return;
  }
  launch_fwd_t<OUT_BF16, 128, 128, 2>(s, ac, as, ats, apg, bc, bs, bts, off, E, M, N, K, c);
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

extern "C" int moe_grouped_gemm_fwd_hmx8(const uint8_t* a_codes, const uint8_t* a_sf, const float* a_ts,
                                         int a_ts_per_group, const uint8_t* b_codes, const uint8_t* b_sf,
                                         const float* b_ts, const int32_t* expert_off, int32_t E, int64_t M_total,
                                         int64_t N, int64_t K, float* c, int8_t* hcodes, uint8_t* hsf, void* stream) {
  MOE4_REQUIRE(E >= 1 && M_total >= 0 && N > 0 && K > 0, MOE4_EINVAL, "moe_grouped_gemm_fwd_hmx8: bad sizes");
  MOE4_REQUIRE(a_ts && b_codes && b_sf && b_ts && expert_off, MOE4_EINVAL, "moe_grouped_gemm_fwd_hmx8: NULL pointer");
  MOE4_REQUIRE(M_total == 0 || (a_codes && a_sf && c && hcodes && hsf), MOE4_EINVAL,
               "moe_grouped_gemm_fwd_hmx8: NULL pointer");
  MOE4_REQUIRE(aligned16(a_codes) && aligned16(b_codes) && aligned16(c), MOE4_EALIGN,
               "moe_grouped_gemm_fwd_hmx8: misaligned pointer");
  const int choice = fwd_choice(M_total, N, K, E);
  MOE4_REQUIRE(M_total == 0 || choice == 10 || choice == 11, MOE4_EUNSUPPORTED,
               "moe_grouped_gemm_fwd_hmx8: needs the warp-specialised kernels (K % 256 == 0, N % 128 == 0, more "
               "than 32 rows per expert on average)");
  MOE4_REQUIRE(M_total * N < ((int64_t)1 << 32), MOE4_EINVAL, "moe_grouped_gemm_fwd_hmx8: payload too large");
  if (M_total == 0) return MOE4_OK;
  MOE4_REQUIRE(((N + 127) / 128) * ((M_total + 127) / 128 + E) < ((int64_t)1 << 31), MOE4_EINVAL,
               "moe_grouped_gemm_fwd_hmx8: too large");
  hipStream_t s = as_stream(stream);
  if (choice == 11)
    hipLaunchKernelGGL((k_gemm_fwd_ws<false, 256, true>), dim3((unsigned)fws_grid()), dim3(fws::Cfg<256>::NT), 0, s,
                       a_codes, a_sf, a_ts, a_ts_per_group, b_codes, b_sf, b_ts, expert_off, E, M_total, N, K,
                       dg_split(N / 256, fws::TM, 256), static_cast<void*>(c), nullptr, nullptr, hcodes, hsf);
  else
    hipLaunchKernelGGL((k_gemm_fwd_ws<false, 128, true>), dim3((unsigned)fws_grid()), dim3(fws::Cfg<128>::NT), 0, s,
                       a_codes, a_sf, a_ts, a_ts_per_group, b_codes, b_sf, b_ts, expert_off, E, M_total, N, K,
                       dg_split(N / 128, fws::TM, 128), static_cast<void*>(c), nullptr, nullptr, hcodes, hsf);
  return check_launch("moe_grouped_gemm_fwd_hmx8");
}

namespace moe4 {
__global__ void k_zero_amax(uint32_t* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}
}  // namespace moe4

extern "C" int moe_grouped_gemm_fwd_silu_amax(const uint8_t* a_codes, const uint8_t* a_sf, const float* a_ts,
                                              int a_ts_per_group, const uint8_t* b_codes, const uint8_t* b_sf,
                                              const float* b_ts, const int32_t* expert_off, int32_t E, int64_t M_total,
                                              int64_t N, int64_t K, uint16_t* c, uint32_t* silu_amax, void* stream) {
  MOE4_REQUIRE(E >= 1 && M_total >= 0 && N > 0 && K > 0, MOE4_EINVAL, "moe_grouped_gemm_fwd_silu_amax: bad sizes");
  MOE4_REQUIRE(K % 64 == 0 && N % 32 == 0, MOE4_EINVAL,
               "moe_grouped_gemm_fwd_silu_amax: need K % 64 == 0 and N % 32 == 0");
  MOE4_REQUIRE(a_ts && b_codes && b_sf && b_ts && expert_off && silu_amax, MOE4_EINVAL,
               "moe_grouped_gemm_fwd_silu_amax: NULL pointer");
  MOE4_REQUIRE(M_total == 0 || (a_codes && a_sf && c), MOE4_EINVAL, "moe_grouped_gemm_fwd_silu_amax: NULL pointer");
  MOE4_REQUIRE(aligned16(a_codes) && aligned16(b_codes) && aligned16(c), MOE4_EALIGN,
               "moe_grouped_gemm_fwd_silu_amax: misaligned pointer");
  const int choice = fwd_choice(M_total, N, K, E);
  MOE4_REQUIRE(M_total == 0 || choice == 10 || choice == 11 || choice == 12, MOE4_EUNSUPPORTED,
               "moe_grouped_gemm_fwd_silu_amax: needs the warp-specialised or few-rows kernels (K % 256 == 0, "
               "N % 128 == 0, or N % 64 == 0 with at most 32 rows per expert on average)");
  MOE4_REQUIRE(((N + 127) / 128) * ((M_total + 127) / 128 + E) < ((int64_t)1 << 31), MOE4_EINVAL,
               "moe_grouped_gemm_fwd_silu_amax: too large");
  hipStream_t s = as_stream(stream);
  const float* tab = nullptr;
  int rc = act_tables(&tab);
  if (rc) return rc;
  hipLaunchKernelGGL(k_zero_amax, dim3((E + 255) / 256), dim3(256), 0, s, silu_amax, E);
  if (M_total == 0) return check_launch("moe_grouped_gemm_fwd_silu_amax");
  launch_fwd<true>(s, a_codes, a_sf, a_ts, a_ts_per_group, b_codes, b_sf, b_ts, expert_off, E, M_total, N, K, c,
                   silu_amax, tab);
  return check_launch("moe_grouped_gemm_fwd_silu_amax");
}
