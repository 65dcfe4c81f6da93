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
// K block g.
//
// Kernel shape: BM x BN tile, K slabs of 64 bytes (one MFMA step), 256
// threads as 2 x 2 waves of (BM/2) x (BN/2).  Operands are read with raw
// buffer loads (32-bit offsets from a per-operand descriptor whose range check
// returns zeros past the tensor and for masked K tails, so no load branches);
// the whole slab's MFMA operands are held in registers; slab s is fetched
// into one of two register sets three slabs ahead, written to LDS one slab
// ahead (LDS rows unpadded with XOR-swizzled 16-byte chunks: conflict-free
// slab writes and fragment reads), and its MFMAs overlap the next slab's LDS
// traffic.
#include <stdlib.h>

#include <type_traits>

#include "gemm_common.h"
#include "moe4_internal.h"

namespace moe4 {

namespace bwd {
constexpr int THREADS = 256;
constexpr int BK = 64;
constexpr int LDS_STRIDE = BK;  // bytes per LDS row: unpadded, 16-byte chunks XOR-swizzled by row
// physical 16-byte chunk of logical chunk c in row r: a wave's 64 slab writes
// fill 1 KB contiguously and 16 lanes reading one logical chunk of 16
// consecutive rows hit 16 distinct 4-bank groups
__device__ inline int swz(int r, int c) { return c ^ ((r >> 2) & 3); }
constexpr uint32_t OOB = 0x80000000u;  // offset past every operand: loads return 0
}  // namespace bwd

// Workgroup barrier that the scheduler may not move any instruction across
// (plain __syncthreads() lets MFMAs, which touch no memory, sink past it).
__device__ __forceinline__ void pinned_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();
  __builtin_amdgcn_sched_barrier(0);
}


// One operand's slab in registers: ROWS rows x 64 bytes, NT threads.  Thread
// t loads the 16-byte chunk t % 4 of rows t / 4 + (NT / 4) j, and the 2 scale
// bytes of row t (t < ROWS).  Scales are row-major [rows][ld/32] or, with
// sf_blocks, block-major [ld/32][rows].
template <int ROWS, int NT>
struct MxSlab {
  static constexpr int NQ = ROWS * 4 / NT;
  u32x4 q[NQ];
  uint32_t s0, s1;  // scale bytes of K blocks 0 and 1 (combined only when written to LDS)
};

template <int ROWS, int NT>
struct MxOperand {
  static constexpr int NQ = ROWS * 4 / NT;
  __amdgpu_buffer_rsrc_t codes, scales;
  uint32_t off[NQ];  // byte offset of the thread's rows (k excluded)
  uint32_t soff;     // byte offset of the thread's row's first scale (t < ROWS)
  uint32_t sbs;      // byte stride between consecutive K blocks of a row's scales
  uint32_t klen;

  __device__ void init(const uint8_t* c, const uint8_t* s, int64_t rows_total, int64_t ld, int64_t row0, int64_t kl,
                       bool sf_blocks = false) {
    codes = make_rsrc(c, (uint64_t)rows_total * ld);
    scales = make_rsrc(s, (uint64_t)rows_total * (ld / 32));
    klen = (uint32_t)kl;
    const int t = threadIdx.x;
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      const int64_t row = row0 + t / 4 + (NT / 4) * j;
      off[j] = row < rows_total ? (uint32_t)(row * ld + (t % 4) * 16) : bwd::OOB;
    }
    const int64_t row = row0 + t;
    soff = (t < ROWS && row < rows_total) ? (uint32_t)(sf_blocks ? row : row * (ld / 32)) : bwd::OOB;
    sbs = sf_blocks ? (uint32_t)rows_total : 1u;
  }

  // k0 past the contraction yields zeros (the descriptor's range check).
  __device__ void load(MxSlab<ROWS, NT>& r, uint32_t k0) const {
    const int t = threadIdx.x;
    const bool kok = k0 + (t % 4) * 16 < klen;
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      const uint32_t o = (kok && off[j] != bwd::OOB) ? off[j] + k0 : bwd::OOB;
      r.q[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(codes, o, 0, 0));
    }
    const uint32_t so = (soff == bwd::OOB || k0 >= klen) ? bwd::OOB : soff + (k0 / 32) * sbs;
    r.s0 = __builtin_amdgcn_raw_buffer_load_b8(scales, so, 0, 0);
    r.s1 = __builtin_amdgcn_raw_buffer_load_b8(scales, (k0 + 32 < klen && so != bwd::OOB) ? so + sbs : bwd::OOB, 0, 0);
  }
};

// Scale bytes go to LDS as [part h][block b][lane row li][fragment f] with
// row = h * ROWS/PARTS + 32 f + li (PARTS = waves along this operand's
// rows), so a lane reads the scales of all its fragments for one K block
// with one small LDS read.
template <int ROWS, int NT, int PARTS>
__device__ inline void store_mx_slab(const MxSlab<ROWS, NT>& r, uint8_t* lds, uint8_t* lds_s) {
  constexpr int F = ROWS / (32 * PARTS);  // 32-row fragments per part
  const int t = threadIdx.x;
#pragma unroll
  for (int j = 0; j < MxSlab<ROWS, NT>::NQ; ++j) {
    const int row = t / 4 + (NT / 4) * j;
    *reinterpret_cast<u32x4*>(lds + row * bwd::LDS_STRIDE + bwd::swz(row, t % 4) * 16) = r.q[j];
  }
  if (NT <= ROWS || t < ROWS) {  // (no branch when every thread has a row: keeps the step one basic block)
    const int h = t / (ROWS / PARTS), f = (t % (ROWS / PARTS)) / 32, li = t % 32;
    lds_s[((h * 2 + 0) * 32 + li) * F + f] = (uint8_t)r.s0;
    lds_s[((h * 2 + 1) * 32 + li) * F + f] = (uint8_t)r.s1;
  }
}

// F scale bytes (one per fragment) from LDS as one integer, byte f = fragment f.
template <int F>
__device__ inline uint32_t lds_scale_bytes(const uint8_t* p) {
  if (F == 4) return *reinterpret_cast<const uint32_t*>(p);
  if (F == 2) return *reinterpret_cast<const uint16_t*>(p);
  return *p;
}

// Per-workgroup MFMA machinery shared by the two kernels, as a macro of
// lambdas over the kernel's locals (fragments, accumulators, LDS pointers):
// one slab in LDS, the wave's fragments of it in registers.  WVM x WVN waves
// of (BM/WVM) x (BN/WVN).  In the 32x32 MFMA layout lane l holds, for value
// v, row (v/4)*8 + (l/32)*4 + v%4 and column l%32 of the fragment, so each
// epilogue store instruction writes two full 128-byte row segments
// (partial-line stores cost far more).
#define MOE4_MX_CORE(BM, BN, WVM, WVN, NBUF)                                                                      \
  constexpr int NT = 64 * (WVM) * (WVN);                                                                       \
  constexpr int WM = (BM) / (WVM), MI = WM / 32, WN = (BN) / (WVN), NJ = WN / 32;                              \
  constexpr int A_BYTES = (BM) * bwd::LDS_STRIDE, B_BYTES = (BN) * bwd::LDS_STRIDE;                            \
  constexpr int STAGE = A_BYTES + B_BYTES + ((BM) + (BN)) * 2;                                                 \
  __shared__ __attribute__((aligned(16))) uint8_t smem[STAGE * (NBUF)];                                      \
  uint8_t* const la = smem;                                                                                    \
  uint8_t* const lb = smem + A_BYTES;                                                                          \
  uint8_t* const las = smem + A_BYTES + B_BYTES;                                                               \
  uint8_t* const lbs = las + (BM) * 2;                                                                         \
  const int w = threadIdx.x >> 6, g = (threadIdx.x >> 5) & 1, li = threadIdx.x & 31;                           \
  const int wmi = w / (WVN), wni = w % (WVN);                                                                  \
  const int wm = wmi * WM, wn = wni * WN;                                                                      \
  f32x16 acc[MI][NJ];                                                                                          \
  i32x8 fa[MI], fb[NJ];                                                                                        \
  int sa[MI], sb[NJ];                                                                                          \
  auto zero_acc = [&]() {                                                                                      \
    _Pragma("unroll") for (int i = 0; i < MI; ++i) _Pragma("unroll") for (int j = 0; j < NJ; ++j) acc[i][j] =   \
        f32x16{};                                                                                              \
  };                                                                                                           \
  auto stage = [&](const MxSlab<BM, NT>& ra, const MxSlab<BN, NT>& rb) {                                       \
    store_mx_slab<BM, NT, WVM>(ra, la, las);                                                                   \
    store_mx_slab<BN, NT, WVN>(rb, lb, lbs);                                                                   \
  };                                                                                                           \
  auto read_frags = [&]() {                                                                                    \
    const uint32_t sa_w = lds_scale_bytes<MI>(las + ((wmi * 2 + g) * 32 + li) * MI);                          \
    const uint32_t sb_w = lds_scale_bytes<NJ>(lbs + ((wni * 2 + g) * 32 + li) * NJ);                          \
    _Pragma("unroll") for (int i = 0; i < MI; ++i) {                                                           \
      const int r = wm + i * 32 + li;                                                                          \
      const uint8_t* p = la + r * bwd::LDS_STRIDE;                                                             \
      i32x4 x0 = *reinterpret_cast<const i32x4*>(p + 16 * bwd::swz(r, g));                                     \
      i32x4 x1 = *reinterpret_cast<const i32x4*>(p + 16 * bwd::swz(r, 2 + g));                                 \
      fa[i] = i32x8{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};                                   \
      sa[i] = (sa_w >> (8 * i)) & 0xFF;                                                                        \
    }                                                                                                          \
    _Pragma("unroll") for (int j = 0; j < NJ; ++j) {                                                           \
      const int r = wn + j * 32 + li;                                                                          \
      const uint8_t* p = lb + r * bwd::LDS_STRIDE;                                                             \
      i32x4 x0 = *reinterpret_cast<const i32x4*>(p + 16 * bwd::swz(r, g));                                     \
      i32x4 x1 = *reinterpret_cast<const i32x4*>(p + 16 * bwd::swz(r, 2 + g));                                 \
      fb[j] = i32x8{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};                                   \
      sb[j] = (sb_w >> (8 * j)) & 0xFF;                                                                        \
    }                                                                                                          \
  };                                                                                                           \
  auto mfmas = [&]() {                                                                                         \
    _Pragma("unroll") for (int i = 0; i < MI; ++i) _Pragma("unroll") for (int j = 0; j < NJ; ++j) acc[i][j] =   \
        __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[i], fb[j], acc[i][j], 0, 0, 0, sa[i], 0, sb[j]);   \
  };                                                                                                           \
  /* C[row0 + r][n0 + c] (+)= tile; rows >= row_end, columns >= N skipped  */                                  \
  auto store_tile = [&](float* C, int64_t ldc, int64_t row0, int64_t row_end, int64_t n0, int64_t N,          \
                        float beta) {                                                                          \
    _Pragma("unroll") for (int i = 0; i < MI; ++i) _Pragma("unroll") for (int j = 0; j < NJ; ++j) {            \
      const int64_t col = n0 + wn + j * 32 + li;                                                               \
      _Pragma("unroll") for (int v = 0; v < 16; ++v) {                                                         \
        const int64_t row = row0 + wm + i * 32 + (v >> 2) * 8 + g * 4 + (v & 3);                              \
        if (row < row_end && col < N) {                                                                        \
          float* p = C + row * ldc + col;                                                                      \
          float val = acc[i][j][v];                                                                            \
          if (beta != 0.0f) val = *p + val;                                                                    \
          __builtin_nontemporal_store(val, p);                                                                 \
        }                                                                                                      \
      }                                                                                                        \
    }                                                                                                          \
  };                                                                                                           \
  /* zeros over the same region: each wave writes whole rows of its part,  */                                  \
  /* 16 bytes per lane                                                      */                                  \
  auto zero_tile = [&](float* C, int64_t ldc, int64_t row0, int64_t row_end, int64_t n0, int64_t N) {          \
    constexpr int LPR = WN / 4; /* lanes per row */                                                            \
    _Pragma("unroll") for (int k = 0; k < WM * LPR / 64; ++k) {                                                \
      const int idx = k * 64 + (threadIdx.x & 63);                                                             \
      const int64_t row = row0 + wm + idx / LPR, col = n0 + wn + (idx % LPR) * 4;                              \
      if (row < row_end && col < N)                                                                            \
        __builtin_nontemporal_store(f32x4{0.f, 0.f, 0.f, 0.f}, reinterpret_cast<f32x4*>(C + row * ldc + col)); \
    }                                                                                                          \
  };                                                                                                           \
  zero_acc()

// dgrad: A [M_total][K] with rows grouped by expert_off, B [E][N][K],
// C [M_total][N].  One workgroup per tile (XCD-aware order, N tile fastest:
// every M tile holds up to BM rows of one expert, so tiles carry even work).
template <int BM, int BN, int WVM, int WVN, int MINB, int DEPTH>
__global__ void __launch_bounds__(64 * WVM * WVN, MINB) k_dgrad_mx(const uint8_t* __restrict__ a_codes,
                                                                   const uint8_t* __restrict__ a_sf,
                                                                   const uint8_t* __restrict__ b_codes,
                                                                   const uint8_t* __restrict__ b_sf,
                                                                   const int32_t* __restrict__ off, int E,
                                                                   int64_t M_total, int64_t N, int64_t K,
                                                                   int64_t n_ntiles, int64_t n_all,
                                                                   float* __restrict__ c) {
  using namespace bwd;
  const int64_t tile = xcd_tile(blockIdx.x, n_all);
  if (tile >= n_all) return;
  const int64_t nt = tile % n_ntiles;
  int e;
  int64_t mt;
  if (!find_m_tile(off, E, BM, tile / n_ntiles, e, mt)) return;
  const int64_t row0 = (int64_t)off[e] + mt * BM;
  const int64_t row_end = (int64_t)off[e + 1] < M_total ? (int64_t)off[e + 1] : M_total;
  const int64_t n0 = nt * BN;
  MOE4_MX_CORE(BM, BN, WVM, WVN, (DEPTH == 4 ? 2 : 1));
  MxOperand<BM, NT> opa;
  MxOperand<BN, NT> opb;
  opa.init(a_codes, a_sf, M_total, K, row0, K);
  opb.init(b_codes + (int64_t)e * N * K, b_sf + (int64_t)e * N * (K / 32), N, K, n0, K);
  const uint32_t nk = (uint32_t)((K + BK - 1) / BK);
  if (DEPTH == 3) {
    // Slab s is loaded into register set s % 2 three slabs ahead, written to
    // LDS one slab ahead, and read into the fragment registers right after
    // the previous slab's MFMAs.  Past the last slab the loads return zeros
    // and the LDS traffic is unused, so the body has no branches.
    MxSlab<BM, NT> ra0, ra1;
    MxSlab<BN, NT> rb0, rb1;
    auto step = [&](uint32_t s, MxSlab<BM, NT>& ra_next, MxSlab<BN, NT>& rb_next) {
      pinned_barrier();
      stage(ra_next, rb_next);
      opa.load(ra_next, (s + 3) * BK);
      opb.load(rb_next, (s + 3) * BK);
      mfmas();
      pinned_barrier();
      read_frags();
    };
    if (nk > 0) {  // (always; as a branch it keeps the 256 x 256 variant from spilling)
      opa.load(ra0, 0);
      opb.load(rb0, 0);
      stage(ra0, rb0);
      opa.load(ra1, BK);
      opb.load(rb1, BK);
      opa.load(ra0, 2 * BK);
      opb.load(rb0, 2 * BK);
      __syncthreads();
      read_frags();
    }
    uint32_t it = 0;
    for (; it + 1 < nk; it += 2) {
      step(it, ra1, rb1);
      step(it + 1, ra0, rb0);
    }
    if (it < nk) step(it, ra1, rb1);
  } else if (DEPTH == 4) {
    // Double-buffered LDS, one barrier per slab.  Step s: write slab s + 2
    // (register set s % 2) into LDS buffer s % 2 (slab s's fragments were
    // read out at step s - 1), fetch slab s + 4 into that register set, and
    // run slab s's MFMAs while reading slab s + 1's fragments from buffer
    // (s + 1) % 2 into the other fragment set.
    MxSlab<BM, NT> r0a, r1a;
    MxSlab<BN, NT> r0b, r1b;
    i32x8 ga[MI], gb[NJ];
    int tsa[MI], tsb[NJ];
    auto read_into = [&](int buf, i32x8 (&xa)[MI], i32x8 (&xb)[NJ], int (&ya)[MI], int (&yb)[NJ]) {
      const uint8_t* pa = la + buf * STAGE;
      const uint8_t* pb = lb + buf * STAGE;
      const uint32_t sa_w = lds_scale_bytes<MI>(las + buf * STAGE + ((wmi * 2 + g) * 32 + li) * MI);
      const uint32_t sb_w = lds_scale_bytes<NJ>(lbs + buf * STAGE + ((wni * 2 + g) * 32 + li) * NJ);
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        const int r = wm + i * 32 + li;
        const uint8_t* q = pa + r * LDS_STRIDE;
        const i32x4 x0 = *reinterpret_cast<const i32x4*>(q + 16 * swz(r, g));
        const i32x4 x1 = *reinterpret_cast<const i32x4*>(q + 16 * swz(r, 2 + g));
        xa[i] = i32x8{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
        ya[i] = (sa_w >> (8 * i)) & 0xFF;
      }
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int r = wn + j * 32 + li;
        const uint8_t* q = pb + r * LDS_STRIDE;
        const i32x4 x0 = *reinterpret_cast<const i32x4*>(q + 16 * swz(r, g));
        const i32x4 x1 = *reinterpret_cast<const i32x4*>(q + 16 * swz(r, 2 + g));
        xb[j] = i32x8{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
        yb[j] = (sb_w >> (8 * j)) & 0xFF;
      }
    };
    auto mfma_with = [&](const i32x8 (&xa)[MI], const i32x8 (&xb)[NJ], const int (&ya)[MI], const int (&yb)[NJ]) {
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(xa[i], xb[j], acc[i][j], 0, 0, 0, ya[i], 0, yb[j]);
    };
    auto stage_to = [&](int buf, const MxSlab<BM, NT>& xa, const MxSlab<BN, NT>& xb) {
      store_mx_slab<BM, NT, WVM>(xa, la + buf * STAGE, las + buf * STAGE);
      store_mx_slab<BN, NT, WVN>(xb, lb + buf * STAGE, lbs + buf * STAGE);
    };
    // one step; CUR = s % 2 (LDS buffer and register set of slab s + 2)
    auto pstep = [&](uint32_t s, int cur, MxSlab<BM, NT>& xa, MxSlab<BN, NT>& xb, const i32x8 (&fa_c)[MI],
                     const i32x8 (&fb_c)[NJ], const int (&sa_c)[MI], const int (&sb_c)[NJ], i32x8 (&fa_n)[MI],
                     i32x8 (&fb_n)[NJ], int (&sa_n)[MI], int (&sb_n)[NJ]) {
      pinned_barrier();
      stage_to(cur, xa, xb);
      opa.load(xa, (s + 4) * BK);
      opb.load(xb, (s + 4) * BK);
      mfma_with(fa_c, fb_c, sa_c, sb_c);
      read_into(cur ^ 1, fa_n, fb_n, sa_n, sb_n);
#pragma unroll
      for (int k = 0; k < MI * NJ; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
        __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // DS write
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM read
      }
    };
    if (nk > 0) {
      opa.load(r0a, 0);
      opb.load(r0b, 0);
      opa.load(r1a, BK);
      opb.load(r1b, BK);
      stage_to(0, r0a, r0b);
      opa.load(r0a, 2 * BK);
      opb.load(r0b, 2 * BK);
      stage_to(1, r1a, r1b);
      opa.load(r1a, 3 * BK);
      opb.load(r1b, 3 * BK);
      __syncthreads();
      read_into(0, fa, fb, sa, sb);
    }
    uint32_t it = 0;
    for (; it + 1 < nk; it += 2) {
      pstep(it, 0, r0a, r0b, fa, fb, sa, sb, ga, gb, tsa, tsb);
      pstep(it + 1, 1, r1a, r1b, ga, gb, tsa, tsb, fa, fb, sa, sb);
    }
    if (it < nk) pstep(it, 0, r0a, r0b, fa, fb, sa, sb, ga, gb, tsa, tsb);
  } else {
    // One register set: slab s + 2 is loaded while slab s + 1 waits in it to
    // be written to LDS (for layouts with two waves per SIMD, whose second
    // wave covers the shorter lead).
    MxSlab<BM, NT> ra;
    MxSlab<BN, NT> rb;
    if (nk > 0) {
      opa.load(ra, 0);
      opb.load(rb, 0);
      stage(ra, rb);
      opa.load(ra, BK);
      opb.load(rb, BK);
      __syncthreads();
      read_frags();
    }
    for (uint32_t s = 0; s < nk; ++s) {
      __syncthreads();
      stage(ra, rb);
      opa.load(ra, (s + 2) * BK);
      opb.load(rb, (s + 2) * BK);
      mfmas();
      pinned_barrier();
      read_frags();
    }
  }
  store_tile(c, N, row0, row_end, n0, N, 0.0f);
}

// dgrad with direct-to-LDS loads (K % 128 == 0).  256 x 256 tile, K slabs of
// 128 bytes (two MFMA steps), two LDS buffers.  Each load instruction of a
// wave fills 1 KB of LDS (lane i -> bytes 16 i .. 16 i + 15), i.e. 8 rows of
// 128 bytes: whole cache lines per row.  Rows keep their 16-byte chunks
// XOR-swizzled by (row >> 1) & 7, so the 16 lanes of a b128 fragment read
// (16 consecutive rows, one logical chunk) hit 16 distinct 4-bank groups;
// the swizzle is applied through the global address each lane fetches.  The
// 4 scale bytes of a row (the slab's 4 K blocks) arrive as one dword.  One
// barrier per slab: after it the next slab's loads are issued into the other
// buffer, and they land while this slab's 32 MFMAs per wave run.  Rows past
// the operands are clamped to the last row (valid memory; their results are
// never stored), so no load is out of range.
namespace dmag {
constexpr int BM = 256, BN = 256, BK = 128, NT = 256;  // (BM, BN: the wgrad variant's tile)
constexpr int CODE = 256 * BK;  // bytes per operand per buffer (256-row tiles)
__device__ inline int swz(int row, int c) { return c ^ ((row >> 1) & 7); }
typedef __attribute__((address_space(3))) void* lds_ptr;
}  // namespace dmag

// OUT_BF16: C is bf16 (round to nearest even), else float32.
template <int TM, int TN, bool OUT_BF16>
__device__ __forceinline__ void dgrad_dma_body(const uint8_t* __restrict__ a_codes,
                                                          const uint8_t* __restrict__ a_sf,
                                                          const uint8_t* __restrict__ b_codes,
                                                          const uint8_t* __restrict__ b_sf,
                                                          const int32_t* __restrict__ off, int E, int64_t M_total,
                                                          int64_t N, int64_t K, int64_t n_ntiles, int64_t n_all,
                                                          void* __restrict__ c) {
  using namespace dmag;
  constexpr int WM = TM / 2, WN = TN / 2, MI = WM / 32, NJ = WN / 32;
  constexpr int QA = TM / 32, QB = TN / 32;  // 1 KB code loads per wave and slab
  constexpr int SA = TM / 64, SB = TN / 64;  // 64-row scale loads per slab (dealt to the waves)
  __shared__ __attribute__((aligned(16))) uint8_t la0[TM * BK];
  __shared__ __attribute__((aligned(16))) uint8_t lb0[TN * BK];
  __shared__ __attribute__((aligned(16))) uint8_t la1[TM * BK];
  __shared__ __attribute__((aligned(16))) uint8_t lb1[TN * BK];
  __shared__ __attribute__((aligned(16))) uint8_t sa0[TM * 4];
  __shared__ __attribute__((aligned(16))) uint8_t sb0[TN * 4];
  __shared__ __attribute__((aligned(16))) uint8_t sa1[TM * 4];
  __shared__ __attribute__((aligned(16))) uint8_t sb1[TN * 4];
  const int64_t tile = xcd_tile(blockIdx.x, n_all);
  if (tile >= n_all) return;
  const int64_t nt = tile % n_ntiles;
  int e;
  int64_t mt;
  if (!find_m_tile(off, E, TM, tile / n_ntiles, e, mt)) return;
  const int64_t row0 = (int64_t)off[e] + mt * TM;
  const int64_t row_end = (int64_t)off[e + 1] < M_total ? (int64_t)off[e + 1] : M_total;
  const int64_t n0 = nt * TN;
  const int tid = threadIdx.x, l = tid & 63, g = (l >> 5) & 1, li = l & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: LDS bases stay scalar (M0)
  const int wm = (w >> 1) * WM, wn = (w & 1) * WN;
  const uint8_t* Bc = b_codes + (int64_t)e * N * K;
  const uint8_t* Bs = b_sf + (int64_t)e * N * (K / 32);
  const __amdgpu_buffer_rsrc_t rac = make_rsrc(a_codes, (uint64_t)M_total * K);
  const __amdgpu_buffer_rsrc_t ras = make_rsrc(a_sf, (uint64_t)M_total * (K / 32));
  const __amdgpu_buffer_rsrc_t rbc = make_rsrc(Bc, (uint64_t)N * K);
  const __amdgpu_buffer_rsrc_t rbs = make_rsrc(Bs, (uint64_t)N * (K / 32));
  // per-lane source offsets (k excluded): instruction q of wave w fills LDS
  // rows (4 q + w) * 8 + l / 8, physical chunk l % 8
  uint32_t aoff[QA], boff[QB];
#pragma unroll
  for (int q = 0; q < QA; ++q) {
    const int row = (4 * q + w) * 8 + (l >> 3);
    const int64_t ra = row0 + row < M_total ? row0 + row : M_total - 1;
    aoff[q] = (uint32_t)(ra * K + 16 * swz(row, l & 7));
  }
#pragma unroll
  for (int q = 0; q < QB; ++q) {
    const int row = (4 * q + w) * 8 + (l >> 3);
    const int64_t rb = n0 + row < N ? n0 + row : N - 1;
    boff[q] = (uint32_t)(rb * K + 16 * swz(row, l & 7));
  }
  // scale loads: 64 rows (one dword = the slab's 4 blocks each) per
  // instruction; instruction t of the SA + SB is issued by wave t % 4
  uint32_t soff[(SA + SB + 3) / 4];
#pragma unroll
  for (int k = 0; k < (SA + SB + 3) / 4; ++k) {
    const int t = 4 * k + w;
    int64_t r = 0;
    if (t < SA) r = row0 + t * 64 + l < M_total ? row0 + t * 64 + l : M_total - 1;
    else if (t < SA + SB) r = n0 + (t - SA) * 64 + l < N ? n0 + (t - SA) * 64 + l : N - 1;
    soff[k] = (uint32_t)(r * (K / 32));
  }
  auto issue = [&](uint8_t* la, uint8_t* lb, uint8_t* sa, uint8_t* sb, uint32_t k0) {
#pragma unroll
    for (int q = 0; q < QA; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rac, (lds_ptr)(la + (4 * q + w) * 1024), 16, aoff[q] + k0, 0, 0, 0);
#pragma unroll
    for (int q = 0; q < QB; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rbc, (lds_ptr)(lb + (4 * q + w) * 1024), 16, boff[q] + k0, 0, 0, 0);
#pragma unroll
    for (int k = 0; k < (SA + SB + 3) / 4; ++k) {
      const int t = 4 * k + w;  // wave-uniform
      if (t < SA)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ras, (lds_ptr)(sa + t * 256), 4, soff[k] + k0 / 32, 0, 0, 0);
      else if (t < SA + SB)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rbs, (lds_ptr)(sb + (t - SA) * 256), 4, soff[k] + k0 / 32, 0, 0, 0);
    }
  };
  f32x16 acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = f32x16{};
  // 32-row fragments of this wave that hold rows of the expert (small
  // experts leave most of a 256-row tile empty: their MFMAs are skipped)
  const int64_t left = row_end - (row0 + wm);
  const int mi_valid = __builtin_amdgcn_readfirstlane(left <= 0 ? 0 : 1);
  auto compute_n = [&](const uint8_t* la, const uint8_t* lb, const uint8_t* sa, const uint8_t* sb) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      i32x8 fa[MI], fb[NJ];
      int ya[MI], yb[NJ];
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        const int r = wm + i * 32 + li;
        const uint8_t* p = la + r * BK;
        const i32x4 x0 = *reinterpret_cast<const i32x4*>(p + 16 * swz(r, ks * 4 + g));
        const i32x4 x1 = *reinterpret_cast<const i32x4*>(p + 16 * swz(r, ks * 4 + 2 + g));
        fa[i] = i32x8{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
        ya[i] = sa[r * 4 + ks * 2 + g];
      }
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int r = wn + j * 32 + li;
        const uint8_t* p = lb + r * BK;
        const i32x4 x0 = *reinterpret_cast<const i32x4*>(p + 16 * swz(r, ks * 4 + g));
        const i32x4 x1 = *reinterpret_cast<const i32x4*>(p + 16 * swz(r, ks * 4 + 2 + g));
        fb[j] = i32x8{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
        yb[j] = sb[r * 4 + ks * 2 + g];
      }
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[i], fb[j], acc[i][j], 0, 0, 0, ya[i], 0, yb[j]);
    }
  };
  auto compute = [&](const uint8_t* la, const uint8_t* lb, const uint8_t* sa, const uint8_t* sb) {
    if (mi_valid > 0) compute_n(la, lb, sa, sb);
  };
  // Step s: wait for this wave's loads of slab s and its LDS reads of slab
  // s - 1, barrier (everyone's slab s has landed, nobody still reads the
  // other buffer), issue slab s + 1 into the other buffer, compute slab s.
  auto sync = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0);  // vmcnt(0) expcnt(0) lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };
  const uint32_t nk = (uint32_t)(K / BK);
  issue(la0, lb0, sa0, sb0, 0);
  uint32_t s = 0;
  for (; s + 2 <= nk; s += 2) {
    sync();
    issue(la1, lb1, sa1, sb1, (s + 1) * BK);
    compute(la0, lb0, sa0, sb0);
    sync();
    if (s + 2 < nk) issue(la0, lb0, sa0, sb0, (s + 2) * BK);
    compute(la1, lb1, sa1, sb1);
  }
  if (s < nk) {
    sync();
    compute(la0, lb0, sa0, sb0);
  }
  // epilogue: direct stores, two full 128-byte row segments per instruction
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int64_t col = n0 + wn + j * 32 + li;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t row = row0 + wm + i * 32 + (v >> 2) * 8 + g * 4 + (v & 3);
        if (row < row_end && col < N) {
          if (OUT_BF16)
            __builtin_nontemporal_store((uint16_t)f32_to_bf16_bits(acc[i][j][v]),
                                        static_cast<uint16_t*>(c) + row * N + col);
          else
            __builtin_nontemporal_store(acc[i][j][v], static_cast<float*>(c) + row * N + col);
        }
      }
    }
}

// wgrad: per expert e, A_e [N1][P_e] and B_e [N2][P_e] (group-major padded
// transposed MXFP8, contraction over the expert's P_e padded tokens) ->
// dw[e] [N1][N2].  Persistent: workgroup b walks tiles b, b + grid, ... of
// the expert-major tile order (consecutive tiles of one expert land on
// different workgroups, so heavy experts spread over the chip and their
// operands are read while still cached), and feeds one continuous slab
// stream across its tiles: the loads of the next tile's first slabs overlap
// the current tile's last MFMAs and the epilogue stores drain under the
// next tile's work.  Experts without tokens only get their zero tile
// (nothing for beta = 1).
template <int BM, int BN, int WVM, int WVN, int MINB>
__global__ void __launch_bounds__(64 * WVM * WVN, MINB) k_wgrad_mx(const uint8_t* __restrict__ a_codes,
                                                                 const uint8_t* __restrict__ a_sf,
                                                                 const uint8_t* __restrict__ b_codes,
                                                                 const uint8_t* __restrict__ b_sf,
                                                                 const int32_t* __restrict__ off, int E,
                                                                 int64_t N1, int64_t N2, int64_t n_ntiles,
                                                                 int64_t n_all, float* __restrict__ dw,
                                                                 float beta, bool zero_empty) {
  using namespace bwd;
  const int64_t per_e = n_all / E;  // tiles per expert
  const int64_t stride = gridDim.x;
  MOE4_MX_CORE(BM, BN, WVM, WVN, 1);
  // the expert offsets, staged in LDS when they fit (the walk reads them per tile)
  constexpr int OFF_LDS = 2048;
  __shared__ int32_t s_off[OFF_LDS];
  if (E < OFF_LDS) {
    for (int i = threadIdx.x; i <= E; i += NT) s_off[i] = off[i];
    __syncthreads();
  }
  const int32_t* offs = E < OFF_LDS ? s_off : off;
  auto klen_of = [&](int64_t t) {
    const int e = (int)(t / per_e);
    return (int64_t)offs[e + 1] - offs[e];
  };
  // next tile at or after t (in the workgroup's walk) whose expert has
  // tokens; tiles of empty experts met on the way get zeros if fill
  auto next_tile = [&](int64_t t, bool fill) {
    while (t < n_all && klen_of(t) == 0) {
      if (fill && beta == 0.0f && zero_empty) {
        const int e = (int)(t / per_e);
        const int64_t rest = t % per_e;
        zero_tile(dw + (int64_t)e * N1 * N2, N2, (rest / n_ntiles) * BM, N1, (rest % n_ntiles) * BN, N2);
      }
      t += stride;
    }
    return t;
  };
  // load cursor: tile lt, slab ls of lnk
  MxOperand<BM, NT> opa;
  MxOperand<BN, NT> opb;
  int64_t lt = 0;
  uint32_t ls = 0, lnk = 0;
  auto set_load_tile = [&](int64_t t) {
    lt = t;
    ls = 0;
    if (t < n_all) {
      const int e = (int)(t / per_e);
      const int64_t rest = t % per_e;
      const int64_t p0 = offs[e], kl = (int64_t)offs[e + 1] - p0;
      opa.init(a_codes + N1 * p0, a_sf + N1 * p0 / 32, N1, kl, (rest / n_ntiles) * BM, kl, true);
      opb.init(b_codes + N2 * p0, b_sf + N2 * p0 / 32, N2, kl, (rest % n_ntiles) * BN, kl, true);
      lnk = (uint32_t)((kl + BK - 1) / BK);
    } else {  // past the walk: zero-range loads
      opa.klen = 0;
      opb.klen = 0;
      lnk = 0xFFFFFFFFu;
    }
  };
  auto load_next = [&](MxSlab<BM, NT>& ra, MxSlab<BN, NT>& rb) {
    opa.load(ra, ls * BK);
    opb.load(rb, ls * BK);
    if (++ls == lnk) set_load_tile(next_tile(lt + stride, false));
  };
  // compute cursor: tile ct, slab cs of cnk
  int64_t ct = next_tile(blockIdx.x, true);
  if (ct >= n_all) return;
  uint32_t cs = 0, cnk = (uint32_t)((klen_of(ct) + BK - 1) / BK);
  set_load_tile(ct);
  MxSlab<BM, NT> ra0, ra1;
  MxSlab<BN, NT> rb0, rb1;
  if (cnk > 0) {  // (always; as a branch it eases register allocation)
    load_next(ra0, rb0);
    stage(ra0, rb0);
    load_next(ra1, rb1);
    load_next(ra0, rb0);
    __syncthreads();
    read_frags();
  }
  // one slab: write slab s+1 to LDS, fetch slab s+3, MFMAs of slab s, read
  // slab s+1; after a tile's last slab, its epilogue
  auto step = [&](MxSlab<BM, NT>& ra_next, MxSlab<BN, NT>& rb_next) -> bool {
    pinned_barrier();
    stage(ra_next, rb_next);
    load_next(ra_next, rb_next);
    mfmas();
    pinned_barrier();
    read_frags();
    if (++cs == cnk) {
      const int e = (int)(ct / per_e);
      const int64_t rest = ct % per_e;
      store_tile(dw + (int64_t)e * N1 * N2, N2, (rest / n_ntiles) * BM, N1, (rest % n_ntiles) * BN, N2, beta);
      zero_acc();
      ct = next_tile(ct + stride, true);
      if (ct >= n_all) return false;
      cs = 0;
      cnk = (uint32_t)((klen_of(ct) + BK - 1) / BK);
    }
    return true;
  };
  while (step(ra1, rb1) && step(ra0, rb0)) {
  }
}

// One kernel per configuration (the body is a device template).
#define MOE4_DGRAD_DMA_KERNEL(NAME, TM, TN, MINB, BF16)                                                            \
  __global__ void __launch_bounds__(dmag::NT, MINB)                                                               \
      NAME(const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_sf,                                 \
           const uint8_t* __restrict__ b_codes, const uint8_t* __restrict__ b_sf, const int32_t* __restrict__ off, \
           int E, int64_t M_total, int64_t N, int64_t K, int64_t n_ntiles, int64_t n_all, void* __restrict__ c) {  \
    dgrad_dma_body<TM, TN, BF16>(a_codes, a_sf, b_codes, b_sf, off, E, M_total, N, K, n_ntiles, n_all, c);       \
  }
MOE4_DGRAD_DMA_KERNEL(k_dgrad_dma_256, 256, 256, 1, false)
MOE4_DGRAD_DMA_KERNEL(k_mx_gemm_dma_256_bf16, 256, 256, 1, true)
#undef MOE4_DGRAD_DMA_KERNEL

// wgrad, warp-specialized and persistent.  On this architecture one
// counter tracks a wave's loads and stores together and completes them in
// issue order, so a wave that both stores a finished tile and waits for its
// next slab's loads waits for the stores' write acknowledgements too: with
// tiles of a few slabs that stall dominates.  Here the roles are split:
// four producer waves only issue direct-to-LDS loads (codes as whole
// 128-byte row segments; the block-major scales of a slab's 4 K blocks x 64
// rows as one dword load) into a ring of S stages,
// and four consumer waves only read LDS, run the MFMAs and store the
// finished tiles, so no load wait ever queues behind a store.  One barrier
// per slab: after barrier g the consumers compute slab g from stage g % S
// while the producers fill stage (g - 1) % S (read by everyone before the
// barrier) with slab g + S - 1, then wait for slab g + 1 to land.  Both
// roles walk the same tiles (b, b + grid, ... of the expert-major order) and
// slab counts, so their barrier counts agree.  Within an expert the column
// blocks run fastest, so concurrently running workgroups write whole rows of
// dW between them (ordering by the larger dimension instead cuts the
// operands' per-XCD re-fetch but scatters the writes, which measured slower); tiles of experts without
// tokens are zero-filled by the consumers (beta = 0) without a barrier.
// K tails, and rows past N1 or N2, come as zeros from out-of-range loads.
namespace wsg {
constexpr int TM = 128, TN = 128, BK = 128, S = 4;
constexpr int NCW = 4, NPW = 4, NT = 64 * (NCW + NPW);
constexpr int CODE = TM * BK;   // one operand's codes per stage
constexpr int SCL = 4 * TM;     // one operand's scale bytes per stage: [row half][K block][64 rows]
constexpr int STAGE = 2 * CODE + 2 * SCL;
constexpr int I = 9;            // loads per producer wave and slab: 8 code row groups + 1 for the scales
// s_waitcnt immediates (vmcnt: bits 3:0 and 15:14; expcnt 6:4; lgkmcnt 11:8)
constexpr int wait_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
constexpr int WAIT_LGKM0 = 15 | (3 << 14) | (7 << 4);
constexpr int MAX_E = 2048;     // expert offsets staged in LDS
constexpr int NT_STORE = 2;     // buffer-store cache policy: nontemporal
}  // namespace wsg

__global__ void __launch_bounds__(wsg::NT, 1)
    k_wgrad_ws(const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_sf,
               const uint8_t* __restrict__ b_codes, const uint8_t* __restrict__ b_sf,
               const int32_t* __restrict__ off, int E, int64_t N1, int64_t N2, int64_t n_ntiles_, int64_t n_all_,
               float* __restrict__ dw, float beta, bool zero_empty) {
  using namespace wsg;
  using dmag::lds_ptr;
  using dmag::swz;
  __shared__ __attribute__((aligned(16))) uint8_t ring[S * STAGE];
  __shared__ int32_t s_off[MAX_E + 1];
  // tile indices fit 31 bits (checked at launch): 32-bit index arithmetic
  const uint32_t n_all = (uint32_t)n_all_, n_ntiles = (uint32_t)n_ntiles_, per_e = n_all / (uint32_t)E;
  // tile rest (within its expert) -> (row block, column block)
  auto tile_mn = [&](uint32_t rest, uint32_t& mt, uint32_t& nt) {
    mt = rest / n_ntiles;
    nt = rest - mt * n_ntiles;
  };
  const int tid = threadIdx.x, l = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  for (int i = tid; i <= E; i += NT) s_off[i] = off[i];
  __syncthreads();
  if (w >= NCW) {
    // ---- producer: wave pw loads half h of operand B (pw >= 2) or A
    const int pw = w - NCW, h = pw & 1;
    const bool opb = pw >= 2;
    const int64_t NR = opb ? N2 : N1;
    const uint8_t* codes = opb ? b_codes : a_codes;
    const uint8_t* sf = opb ? b_sf : a_sf;
    uint32_t pt = blockIdx.x;
    uint32_t ps = 0, pnk = 0, klen = 0, srow = 0;
    uint32_t crow[8];
    __amdgpu_buffer_rsrc_t rc = make_rsrc(codes, 0), rs = make_rsrc(sf, 0);
    // move to the first tile at or after pt whose expert has tokens
    auto seek = [&]() -> bool {
      for (; pt < n_all; pt += gridDim.x) {
        // (offsets from global memory through the scalar cache: an LDS read
        // here would make the compiler wait for this wave's direct-to-LDS loads)
        const uint32_t e = pt / per_e, rest = pt - e * per_e;
        const int64_t p0 = off[e], kl = (int64_t)off[e + 1] - p0;
        if (kl == 0) continue;
        uint32_t mt, nt;
        tile_mn(rest, mt, nt);
        const int64_t r0 = opb ? (int64_t)nt * TN : (int64_t)mt * TM;
        rc = make_rsrc(codes + NR * p0, (uint64_t)NR * kl);
        rs = make_rsrc(sf + NR * p0 / 32, (uint64_t)NR * (kl / 32));
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int row = h * 64 + j * 8 + (l >> 3);
          const uint32_t r = (uint32_t)(r0 + row < NR ? r0 + row : NR - 1);
          crow[j] = r * (uint32_t)kl + 16u * (uint32_t)swz(row, l & 7);
        }
        // lane l: rows r0 + h * 64 + 4 (l % 16) .. + 3 of K block l / 16 of
        // the slab (block-major scales; NR % 32 == 0 keeps the 4 rows together)
        const int64_t rr = r0 + h * 64 + (l & 15) * 4;
        srow = rr < NR ? (uint32_t)((l >> 4) * NR + rr) : bwd::OOB;
        klen = (uint32_t)kl;
        pnk = (uint32_t)((kl + BK - 1) / BK);
        ps = 0;
        return true;
      }
      return false;
    };
    bool more = seek();
    // issue the cursor's slab into stage st and advance the cursor
    auto issue = [&](int st) {
      uint8_t* base = ring + st * STAGE;
      uint8_t* cb = base + (opb ? CODE : 0) + h * 8 * 1024;
      uint8_t* sb = base + 2 * CODE + (opb ? SCL : 0) + h * 256;
      const uint32_t k0 = ps * BK;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const bool ok = k0 + 16 * (uint32_t)swz(h * 64 + j * 8 + (l >> 3), l & 7) < klen;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rc, (lds_ptr)(cb + j * 1024), 16, ok ? crow[j] + k0 : bwd::OOB, 0, 0,
                                                 0);
      }
      const bool sok = srow != bwd::OOB && k0 + 32 * (uint32_t)(l >> 4) < klen;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr)sb, 4, sok ? srow + (k0 / 32) * (uint32_t)NR : bwd::OOB, 0,
                                               0, 0);
      if (++ps == pnk) {
        pt += gridDim.x;
        more = seek();
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
  // ---- consumers: wave w owns the 64 x 64 quadrant (w / 2, w % 2)
  constexpr int MI = 2, NJ = 2;
  const int g = (l >> 5) & 1, li = l & 31;
  const int wm = (w >> 1) * 64, wn = (w & 1) * 64;
  f32x16 acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = f32x16{};
  auto compute = [&](const uint8_t* base) {
    const uint8_t* la = base;
    const uint8_t* lb = base + CODE;
    const uint8_t* sa = base + 2 * CODE;
    const uint8_t* sb = base + 2 * CODE + SCL;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      i32x8 fa[MI], fb[NJ];
      int ya[MI], yb[NJ];
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        const int r = wm + i * 32 + li;
        const uint8_t* p = la + r * BK;
        const i32x4 x0 = *reinterpret_cast<const i32x4*>(p + 16 * swz(r, ks * 4 + g));
        const i32x4 x1 = *reinterpret_cast<const i32x4*>(p + 16 * swz(r, ks * 4 + 2 + g));
        fa[i] = i32x8{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
        ya[i] = sa[(r >> 6) * 256 + (ks * 2 + g) * 64 + (r & 63)];
      }
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int r = wn + j * 32 + li;
        const uint8_t* p = lb + r * BK;
        const i32x4 x0 = *reinterpret_cast<const i32x4*>(p + 16 * swz(r, ks * 4 + g));
        const i32x4 x1 = *reinterpret_cast<const i32x4*>(p + 16 * swz(r, ks * 4 + 2 + g));
        fb[j] = i32x8{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
        yb[j] = sb[(r >> 6) * 256 + (ks * 2 + g) * 64 + (r & 63)];
      }
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[i], fb[j], acc[i][j], 0, 0, 0, ya[i], 0, yb[j]);
    }
  };
  uint32_t gs = 0;  // slab of the stream
  // output stores: buffer stores off one per-lane offset (row g * 4, column
  // li of a fragment) plus a uniform offset per value; N1 and N2 are
  // multiples of 32, so each 32 x 32 fragment is wholly inside or outside
  const uint32_t ld = (uint32_t)N2 * 4;  // row pitch in bytes
  const uint32_t lane_off = (uint32_t)(g * 4) * ld + (uint32_t)li * 4;
  for (uint32_t t = blockIdx.x; t < n_all; t += gridDim.x) {
    const uint32_t e = t / per_e, rest = t - e * per_e;
    uint32_t mt, nt;
    tile_mn(rest, mt, nt);
    const int64_t m0 = (int64_t)mt * TM, c0 = (int64_t)nt * TN;
    const int kl = s_off[e + 1] - s_off[e];
    float* C = dw + (int64_t)e * N1 * N2;
    const __amdgpu_buffer_rsrc_t rC = make_rsrc(C, (uint64_t)N1 * N2 * 4);
    if (kl == 0) {  // no tokens: zeros for beta = 0 (unless skipped); 4 rows x 64 columns per store
      if (beta != 0.0f || !zero_empty) continue;
      const bool cok = c0 + wn + (l & 15) * 4 < N2;
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const int64_t row = m0 + wm + k * 4 + (l >> 4);
        const uint32_t o = (uint32_t)(row * N2 + c0 + wn + (l & 15) * 4) * 4;
        __builtin_amdgcn_raw_buffer_store_b128((__attribute__((ext_vector_type(4))) unsigned){0u, 0u, 0u, 0u}, rC,
                                               row < N1 && cok ? o : bwd::OOB, 0, NT_STORE);
      }
      continue;
    }
    const uint32_t nk = (uint32_t)((kl + BK - 1) / BK);
    for (uint32_t s = 0; s < nk; ++s, ++gs) {
      // this wave's reads of the previous slab are done; barrier g
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(WAIT_LGKM0);
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("" ::: "memory");
      compute(ring + (gs % S) * STAGE);
    }
    // epilogue: two full 128-byte row segments per store instruction
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int64_t r = m0 + wm + i * 32, c = c0 + wn + j * 32;
        if (r < N1 && c < N2) {
          const uint32_t fo = (uint32_t)(r * N2 + c) * 4;
          if (beta == 0.0f) {
#pragma unroll
            for (int v = 0; v < 16; ++v)
              __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[i][j][v]), rC, lane_off,
                                                    fo + (uint32_t)((v >> 2) * 8 + (v & 3)) * ld, NT_STORE);
          } else {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              const uint32_t so = fo + (uint32_t)((v >> 2) * 8 + (v & 3)) * ld;
              const float old = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rC, lane_off, so, 0));
              __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(old + acc[i][j][v]), rC, lane_off, so, NT_STORE);
            }
          }
        }
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
      }
  }
}

// dgrad, warp-specialised and persistent (K % 128 == 0, N % 128 == 0): the
// structure of the forward NVFP4 kernel of this library (four producer waves
// that only issue direct-to-LDS loads into a four-stage ring, four consumer
// waves that only read LDS, run the MFMAs and store; one barrier per slab;
// m-tile-major tiles in contiguous per-XCD runs) with 128 x 128 tiles, so a
// small expert wastes at most 127 padded rows, and the MXFP8 slab of the
// kernel above: 128 code bytes and 4 scale bytes per row and slab, scales
// row-major.  TN = 128 (four stages) or 256 (three stages: consumers of
// 64 x 128, half the operand bytes per MFMA).
namespace dws {
constexpr int TM = 128, NCW = 4, NT = 64 * (NCW + 4);
template <int TN>
struct Cfg {
  static constexpr int CODE_A = TM * dmag::BK, CODE_B = TN * dmag::BK;  // per stage
  static constexpr int SCL_A = TM * 4, SCL_B = TN * 4;
  static constexpr int STAGE = CODE_A + CODE_B + SCL_A + SCL_B;
  static constexpr int S = TN == 128 ? 4 : 3;
  static constexpr int QB = TN / 32;              // B code row groups per producer wave
  static constexpr int NS = TN == 128 ? 1 : 2;    // scale groups per producer wave
  static constexpr int I = 4 + QB + NS;           // loads per producer wave and slab
};
}  // namespace dws

template <bool OUT_BF16, int TN>
__global__ void __launch_bounds__(dws::NT, 1)
    k_dgrad_ws(const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_sf,
               const uint8_t* __restrict__ b_codes, const uint8_t* __restrict__ b_sf,
               const int32_t* __restrict__ off, int E, int64_t M_total, int64_t N, int64_t K, DgSplit sp,
               void* __restrict__ c) {
  using namespace dws;
  using dmag::lds_ptr;
  using dmag::swz;
  using wsg::wait_vm;
  using wsg::WAIT_LGKM0;
  using C = Cfg<TN>;
  constexpr int BK = dmag::BK, S = C::S, STAGE = C::STAGE, I = C::I;
  __shared__ __attribute__((aligned(16))) uint8_t ring[S * STAGE];
  __shared__ uint32_t s_nmt;
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
  const uint32_t n_nt = (uint32_t)(N / TN), n_mt = s_nmt;
  const uint32_t KS = (uint32_t)(K / 32), nk = (uint32_t)(K / BK);
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
    const __amdgpu_buffer_rsrc_t rac = make_rsrc(a_codes, (uint64_t)M_total * K);
    const __amdgpu_buffer_rsrc_t ras = make_rsrc(a_sf, (uint64_t)M_total * KS);
    __amdgpu_buffer_rsrc_t rbc = rac, rbs = ras;
    // (fixed sizes: the first C::QB and C::NS are used; hipcc's host pass rejects
    // arrays sized by the template argument inside the lambdas)
    uint32_t aoff[4], boff[8], soff[2];
    // scale group k of this wave: operand B?, first row
    auto sgrp = [&](int k, bool& opb, int& r0) {
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
      rbc = make_rsrc(b_codes + (int64_t)e * N * K, (uint64_t)N * K);
      rbs = make_rsrc(b_sf + (int64_t)e * N * KS, (uint64_t)N * KS);
      // rows past the operands are clamped to the last row: valid memory whose
      // results are never stored
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = 32 * pw + 8 * q + (l >> 3);
        const int64_t ra = row0 + r < M_total ? row0 + r : M_total - 1;
        aoff[q] = (uint32_t)ra * (uint32_t)K + 16u * (uint32_t)swz(r, l & 7);
      }
#pragma unroll
      for (int q = 0; q < C::QB; ++q) {
        const int r = (TN / 4) * pw + 8 * q + (l >> 3);
        const int64_t rb = n0 + r < N ? n0 + r : N - 1;
        boff[q] = (uint32_t)rb * (uint32_t)K + 16u * (uint32_t)swz(r, l & 7);
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
      const uint32_t kb = ps * (uint32_t)BK, ksb = ps * (uint32_t)(BK / 32);
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
        uint8_t* sb = base + C::CODE_A + C::CODE_B + (opb ? C::SCL_A : 0) + r0 * 4;
        if (opb) __builtin_amdgcn_raw_ptr_buffer_load_lds(rbs, (lds_ptr)sb, 4, soff[k] + ksb, 0, 0, 0);
        else __builtin_amdgcn_raw_ptr_buffer_load_lds(ras, (lds_ptr)sb, 4, soff[k] + ksb, 0, 0, 0);
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
  // ---- consumers: wave w owns the 64 x (TN / 2) block (w / 2, w % 2)
  constexpr int MI = 2, NJ = TN / 64;
  const int g = (l >> 5) & 1, li = l & 31;
  const int wm = (w >> 1) * 64, wn = (w & 1) * (TN / 2);
  f32x16 acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = f32x16{};
  // one slab: two 64-element k steps; lane half g supplies K chunks
  // 4 ks + g and 4 ks + 2 + g and the scale of block 2 ks + g
  auto compute = [&](const uint8_t* base) {
    const uint8_t* la = base;
    const uint8_t* lb = base + C::CODE_A;
    const uint8_t* sa = base + C::CODE_A + C::CODE_B;
    const uint8_t* sb = base + C::CODE_A + C::CODE_B + C::SCL_A;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      i32x8 fa[MI], fb[NJ];
      int ya[MI], yb[NJ];
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        const int r = wm + i * 32 + li;
        const uint8_t* p = la + r * BK;
        const i32x4 x0 = *reinterpret_cast<const i32x4*>(p + 16 * swz(r, ks * 4 + g));
        const i32x4 x1 = *reinterpret_cast<const i32x4*>(p + 16 * swz(r, ks * 4 + 2 + g));
        fa[i] = i32x8{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
        ya[i] = sa[r * 4 + ks * 2 + g];
      }
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int r = wn + j * 32 + li;
        const uint8_t* p = lb + r * BK;
        const i32x4 x0 = *reinterpret_cast<const i32x4*>(p + 16 * swz(r, ks * 4 + g));
        const i32x4 x1 = *reinterpret_cast<const i32x4*>(p + 16 * swz(r, ks * 4 + 2 + g));
        fb[j] = i32x8{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
        yb[j] = sb[r * 4 + ks * 2 + g];
      }
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[i], fb[j], acc[i][j], 0, 0, 0, ya[i], 0, yb[j]);
    }
  };
  constexpr int ESZ = OUT_BF16 ? 2 : 4;
  const uint32_t ld = (uint32_t)N * ESZ;  // output row pitch in bytes
  const uint32_t lane_off = (uint32_t)(g * 4) * ld + (uint32_t)li * ESZ;
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
    // waves whose rows all lie past the expert's last row skip their MFMAs
    const bool active = row0 + wm < row_end;
    for (uint32_t s = 0; s < nk; ++s, ++gs) {
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(WAIT_LGKM0);
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("" ::: "memory");
      if (active) compute(ring + (gs % S) * STAGE);
    }
    // epilogue: each value straight from the accumulators; the descriptor
    // covers the tile's rows up to the expert's last, so stores of rows past
    // it are dropped
    const int64_t nrows = row_end - row0 < TM ? row_end - row0 : TM;
    const __amdgpu_buffer_rsrc_t rC = make_rsrc(static_cast<uint8_t*>(c) + row0 * (int64_t)ld, (uint64_t)nrows * ld);
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        if (active) {
          const uint32_t fo = (uint32_t)(wm + i * 32) * ld + (uint32_t)(n0 + wn + j * 32) * ESZ;
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const uint32_t so = fo + (uint32_t)((v >> 2) * 8 + (v & 3)) * ld;
            if (OUT_BF16)
              __builtin_amdgcn_raw_buffer_store_b16((unsigned short)f32_to_bf16_bits(acc[i][j][v]), rC, lane_off, so,
                                                    wsg::NT_STORE);
            else
              __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[i][j][v]), rC, lane_off, so, wsg::NT_STORE);
          }
        }
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
      }
  }
}

// wgrad with 256 x 128 tiles: k_wgrad_ws's structure, three stages of
// 49.5 KB (A codes 32 KB, B codes 16 KB, scales 1.5 KB: with the offset table,
// all the LDS there is), consumers of 128 x 64.  Each 128-row operand block
// of the 128 x 128 kernel is reloaded for every tile it meets, from L2; the
// wider tile moves three quarters of those bytes per output.  Producer pw
// loads A rows 64 pw .. 64 pw + 63 (8 code row groups + their scales), B rows
// 32 pw .. 32 pw + 31 (4 code row groups) and the scales of B's 64-row half
// pw / 2 (loaded by two waves: every producer issues 14 loads per slab,
// which its waits count).
// An expert's n_mt x n_nt output tiles split into 8 rectangles of pm x pn
// tiles (xa row parts x 8 / xa column parts), one per XCD: virtual tile
// v = 8 q + x is tile q (column fastest) of rectangle x, and workgroup b,
// which runs on XCD b % 8 in a grid that is a multiple of 8, walks the
// tiles b, b + grid, ...: each XCD's L2 then fetches only its rectangle's
// operand rows of the expert instead of nearly all of them.  Virtual tiles
// past the grid (when a dimension does not divide) are skipped.
struct XcdSplit {
  uint32_t n_mt, n_nt, xb, pm, pn;
  __device__ bool tile(uint32_t v, uint32_t& mt, uint32_t& nt) const {
    const uint32_t x = v & 7u, q = v >> 3, px = x / xb, qm = q / pn;
    mt = px * pm + qm;
    nt = (x - px * xb) * pn + (q - qm * pn);
    return mt < n_mt && nt < n_nt;
  }
};

// The split with the fewest operand rows per XCD (counting the virtual
// tiles that fall outside the grid as extra work).
static XcdSplit xcd_split(int64_t n_mt, int64_t n_nt, int tm, int tn) {
  XcdSplit best{};
  double best_cost = 1e300;
  for (uint32_t xa = 1; xa <= 8; xa *= 2) {
    const uint32_t xb = 8 / xa;
    const uint32_t pm = (uint32_t)((n_mt + xa - 1) / xa), pn = (uint32_t)((n_nt + xb - 1) / xb);
    const double rows = (double)pm * tm + (double)pn * tn;
    const double cost = rows * (8.0 * pm * pn) / ((double)n_mt * n_nt);
    if (cost < best_cost) {
      best_cost = cost;
      best = XcdSplit{(uint32_t)n_mt, (uint32_t)n_nt, xb, pm, pn};
    }
  }
  return best;
}

namespace wsg2 {
constexpr int TM = 256, TN = 128, BK = 128, S = 3;
constexpr int CODE_A = TM * BK, CODE_B = TN * BK, SCL_A = 4 * TM, SCL_B = 4 * TN;
constexpr int STAGE = CODE_A + CODE_B + SCL_A + SCL_B;
constexpr int I = 14;
}  // namespace wsg2

__global__ void __launch_bounds__(wsg::NT, 1)
    k_wgrad_ws256(const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_sf,
                  const uint8_t* __restrict__ b_codes, const uint8_t* __restrict__ b_sf,
                  const int32_t* __restrict__ off, int E, int64_t N1, int64_t N2, XcdSplit xs, int64_t n_all_,
                  float* __restrict__ dw, float beta, bool zero_empty) {
  using namespace wsg2;
  using wsg::NCW;
  using wsg::NT;
  using wsg::wait_vm;
  using wsg::WAIT_LGKM0;
  using wsg::MAX_E;
  using wsg::NT_STORE;
  using dmag::lds_ptr;
  using dmag::swz;
  __shared__ __attribute__((aligned(16))) uint8_t ring[S * STAGE];
  __shared__ int32_t s_off[MAX_E + 1];
  const uint32_t n_all = (uint32_t)n_all_, per_e = n_all / (uint32_t)E;
  auto tile_mn = [&](uint32_t rest, uint32_t& mt, uint32_t& nt) { return xs.tile(rest, mt, nt); };
  const int tid = threadIdx.x, l = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  for (int i = tid; i <= E; i += NT) s_off[i] = off[i];
  __syncthreads();
  if (w >= NCW) {
    const int pw = w - NCW, hb = pw >> 1;
    uint32_t pt = blockIdx.x;
    uint32_t ps = 0, pnk = 0, klen = 0, srow_a = 0, srow_b = 0;
    uint32_t crow_a[8], crow_b[4];
    __amdgpu_buffer_rsrc_t rca = make_rsrc(a_codes, 0), rsa = make_rsrc(a_sf, 0);
    __amdgpu_buffer_rsrc_t rcb = rca, rsb = rsa;
    // move to the first tile at or after pt whose expert has tokens
    auto seek = [&]() -> bool {
      for (; pt < n_all; pt += gridDim.x) {
        // (offsets through the scalar unit: an LDS read here would make the
        // compiler wait for this wave's direct-to-LDS loads)
        const uint32_t e = pt / per_e, rest = pt - e * per_e;
        const int64_t p0 = ld_const(off, (int)e), kl = (int64_t)ld_const(off, (int)e + 1) - p0;
        uint32_t mt, nt;
        if (kl == 0 || !tile_mn(rest, mt, nt)) continue;
        const int64_t ra0 = (int64_t)mt * TM, rb0 = (int64_t)nt * TN;
        rca = make_rsrc(a_codes + N1 * p0, (uint64_t)N1 * kl);
        rsa = make_rsrc(a_sf + N1 * p0 / 32, (uint64_t)N1 * (kl / 32));
        rcb = make_rsrc(b_codes + N2 * p0, (uint64_t)N2 * kl);
        rsb = make_rsrc(b_sf + N2 * p0 / 32, (uint64_t)N2 * (kl / 32));
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int row = 64 * pw + 8 * j + (l >> 3);
          const uint32_t r = (uint32_t)(ra0 + row < N1 ? ra0 + row : N1 - 1);
          crow_a[j] = r * (uint32_t)kl + 16u * (uint32_t)swz(row, l & 7);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int row = 32 * pw + 8 * j + (l >> 3);
          const uint32_t r = (uint32_t)(rb0 + row < N2 ? rb0 + row : N2 - 1);
          crow_b[j] = r * (uint32_t)kl + 16u * (uint32_t)swz(row, l & 7);
        }
        // lane l: rows .. + 4 (l % 16) .. + 3 of K block l / 16 of the slab
        // (block-major scales; N1, N2 % 32 == 0 keep the 4 rows together)
        const int64_t rra = ra0 + 64 * pw + (l & 15) * 4, rrb = rb0 + 64 * hb + (l & 15) * 4;
        srow_a = rra < N1 ? (uint32_t)((l >> 4) * N1 + rra) : bwd::OOB;
        srow_b = rrb < N2 ? (uint32_t)((l >> 4) * N2 + rrb) : bwd::OOB;
        klen = (uint32_t)kl;
        pnk = (uint32_t)((kl + BK - 1) / BK);
        ps = 0;
        return true;
      }
      return false;
    };
    bool more = seek();
    auto issue = [&](int st) {
      uint8_t* base = ring + st * STAGE;
      const uint32_t k0 = ps * BK;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const bool ok = k0 + 16 * (uint32_t)swz(64 * pw + 8 * j + (l >> 3), l & 7) < klen;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rca, (lds_ptr)(base + (8 * pw + j) * 1024), 16,
                                                 ok ? crow_a[j] + k0 : bwd::OOB, 0, 0, 0);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bool ok = k0 + 16 * (uint32_t)swz(32 * pw + 8 * j + (l >> 3), l & 7) < klen;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rcb, (lds_ptr)(base + CODE_A + (4 * pw + j) * 1024), 16,
                                                 ok ? crow_b[j] + k0 : bwd::OOB, 0, 0, 0);
      }
      const bool kok = k0 + 32 * (uint32_t)(l >> 4) < klen;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsa, (lds_ptr)(base + CODE_A + CODE_B + pw * 256), 4,
                                               kok && srow_a != bwd::OOB ? srow_a + (k0 / 32) * (uint32_t)N1 : bwd::OOB,
                                               0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsb, (lds_ptr)(base + CODE_A + CODE_B + SCL_A + hb * 256), 4,
                                               kok && srow_b != bwd::OOB ? srow_b + (k0 / 32) * (uint32_t)N2 : bwd::OOB,
                                               0, 0, 0);
      if (++ps == pnk) {
        pt += gridDim.x;
        more = seek();
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
      if (rem >= 1) __builtin_amdgcn_s_waitcnt(wait_vm(I));
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
  // ---- consumers: wave w owns the 128 x 64 block (w / 2, w % 2)
  constexpr int MI = 4, NJ = 2;
  const int g = (l >> 5) & 1, li = l & 31;
  const int wm = (w >> 1) * 128, wn = (w & 1) * 64;
  f32x16 acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = f32x16{};
  auto compute = [&](const uint8_t* base) {
    const uint8_t* la = base;
    const uint8_t* lb = base + CODE_A;
    const uint8_t* sa = base + CODE_A + CODE_B;
    const uint8_t* sb = base + CODE_A + CODE_B + SCL_A;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      i32x8 fa[MI], fb[NJ];
      int ya[MI], yb[NJ];
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        const int r = wm + i * 32 + li;
        const uint8_t* p = la + r * BK;
        const i32x4 x0 = *reinterpret_cast<const i32x4*>(p + 16 * swz(r, ks * 4 + g));
        const i32x4 x1 = *reinterpret_cast<const i32x4*>(p + 16 * swz(r, ks * 4 + 2 + g));
        fa[i] = i32x8{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
        ya[i] = sa[(r >> 6) * 256 + (ks * 2 + g) * 64 + (r & 63)];
      }
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int r = wn + j * 32 + li;
        const uint8_t* p = lb + r * BK;
        const i32x4 x0 = *reinterpret_cast<const i32x4*>(p + 16 * swz(r, ks * 4 + g));
        const i32x4 x1 = *reinterpret_cast<const i32x4*>(p + 16 * swz(r, ks * 4 + 2 + g));
        fb[j] = i32x8{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
        yb[j] = sb[(r >> 6) * 256 + (ks * 2 + g) * 64 + (r & 63)];
      }
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[i], fb[j], acc[i][j], 0, 0, 0, ya[i], 0, yb[j]);
    }
  };
  uint32_t gs = 0;
  const uint32_t ld = (uint32_t)N2 * 4;
  const uint32_t lane_off = (uint32_t)(g * 4) * ld + (uint32_t)li * 4;
  for (uint32_t t = blockIdx.x; t < n_all; t += gridDim.x) {
    const uint32_t e = t / per_e, rest = t - e * per_e;
    uint32_t mt, nt;
    if (!tile_mn(rest, mt, nt)) continue;
    const int64_t m0 = (int64_t)mt * TM, c0 = (int64_t)nt * TN;
    const int kl = s_off[e + 1] - s_off[e];
    float* C = dw + (int64_t)e * N1 * N2;
    const __amdgpu_buffer_rsrc_t rC = make_rsrc(C, (uint64_t)N1 * N2 * 4);
    if (kl == 0) {  // no tokens: zeros for beta = 0 (unless skipped); 4 rows x 64 columns per store
      if (beta != 0.0f || !zero_empty) continue;
      const bool cok = c0 + wn + (l & 15) * 4 < N2;
#pragma unroll 8
      for (int k = 0; k < 32; ++k) {
        const int64_t row = m0 + wm + k * 4 + (l >> 4);
        const uint32_t o = (uint32_t)(row * N2 + c0 + wn + (l & 15) * 4) * 4;
        __builtin_amdgcn_raw_buffer_store_b128((__attribute__((ext_vector_type(4))) unsigned){0u, 0u, 0u, 0u}, rC,
                                               row < N1 && cok ? o : bwd::OOB, 0, NT_STORE);
      }
      continue;
    }
    const uint32_t nk = (uint32_t)((kl + BK - 1) / BK);
    for (uint32_t s = 0; s < nk; ++s, ++gs) {
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(WAIT_LGKM0);
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("" ::: "memory");
      compute(ring + (gs % S) * STAGE);
    }
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int64_t r = m0 + wm + i * 32, c = c0 + wn + j * 32;
        if (r < N1 && c < N2) {
          const uint32_t fo = (uint32_t)(r * N2 + c) * 4;
          if (beta == 0.0f) {
#pragma unroll
            for (int v = 0; v < 16; ++v)
              __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[i][j][v]), rC, lane_off,
                                                    fo + (uint32_t)((v >> 2) * 8 + (v & 3)) * ld, NT_STORE);
          } else {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              const uint32_t so = fo + (uint32_t)((v >> 2) * 8 + (v & 3)) * ld;
              const float old = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rC, lane_off, so, 0));
              __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(old + acc[i][j][v]), rC, lane_off, so, NT_STORE);
            }
          }
        }
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
      }
  }
}

static int cu_count() {
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

template <int BM, int BN, int WVM, int WVN, int MINB, int DEPTH = 3>
static void launch_dgrad_t(const uint8_t* ac, const uint8_t* as, const uint8_t* bc, const uint8_t* bs,
                           const int32_t* off, int E, int64_t M, int64_t N, int64_t K, float* c, hipStream_t s) {
  const int64_t n_nt = (N + BN - 1) / BN;
  const int64_t n_all = n_nt * ((M + BM - 1) / BM + E);
  hipLaunchKernelGGL((k_dgrad_mx<BM, BN, WVM, WVN, MINB, DEPTH>), dim3((unsigned)xcd_grid(n_all)), dim3(64 * WVM * WVN), 0,
                     s, ac, as, bc, bs, off, E, M, N, K, n_nt, n_all, c);
}

template <int BM, int BN, int WVM, int WVN, int MINB>
static void launch_wgrad_t(const uint8_t* ac, const uint8_t* as, const uint8_t* bc, const uint8_t* bs,
                           const int32_t* off, int E, int64_t N1, int64_t N2, float* dw, float beta, bool zero_empty,
                           hipStream_t s) {
  const int64_t n_nt = (N2 + BN - 1) / BN;
  const int64_t n_all = n_nt * ((N1 + BM - 1) / BM) * E;
  int64_t grid = (int64_t)cu_count() * MINB;
  if (grid > n_all) grid = n_all;
  hipLaunchKernelGGL((k_wgrad_mx<BM, BN, WVM, WVN, MINB>), dim3((unsigned)grid), dim3(64 * WVM * WVN), 0, s, ac, as,
                     bc, bs, off, E, N1, N2, n_nt, n_all, dw, beta, zero_empty);
}

// Kernel choice.  dgrad: the warp-specialized persistent kernel with
// 128x256 tiles when K % 128 == 0 and N % 256 == 0, with 128x128 tiles when
// N % 128 == 0; else the direct-to-LDS 256x256 kernel when K % 128 == 0;
// else the register-staged 256x256 kernel (four-deep prefetch).
static void launch_dgrad(const uint8_t* ac, const uint8_t* as, const uint8_t* bc, const uint8_t* bs,
                         const int32_t* off, int E, int64_t M, int64_t N, int64_t K, float* c, hipStream_t s) {
  if (K % dmag::BK == 0 && N % 128 == 0) {
    if (N % 256 == 0)
      hipLaunchKernelGGL((k_dgrad_ws<false, 256>), dim3((unsigned)(cu_count() < 8 ? 8 : cu_count())), dim3(dws::NT), 0, s, ac, as, bc, bs, off,
                         E, M, N, K, dg_split(N / 256, dws::TM, 256), static_cast<void*>(c));
    else
      hipLaunchKernelGGL((k_dgrad_ws<false, 128>), dim3((unsigned)(cu_count() < 8 ? 8 : cu_count())), dim3(dws::NT), 0, s, ac, as, bc, bs, off,
                         E, M, N, K, dg_split(N / 128, dws::TM, 128), static_cast<void*>(c));
    return;
  }
  if (K % dmag::BK == 0) {
    const int64_t n_nt = (N + 255) / 256;
    const int64_t n_all = n_nt * ((M + 255) / 256 + E);
    hipLaunchKernelGGL(k_dgrad_dma_256, dim3((unsigned)xcd_grid(n_all)), dim3(dmag::NT), 0, s, ac, as, bc, bs, off, E,
                       M, N, K, n_nt, n_all, c);
    return;
  }
  launch_dgrad_t<256, 256, 2, 2, 1, 4>(ac, as, bc, bs, off, E, M, N, K, c, s);
}

// wgrad: the warp-specialized persistent kernel with 256x128 tiles, else
// with 128x128 tiles (both need E <= 2048 and 32-bit tile and output
// indices), else the register-staged persistent 128x128 kernel.
static void launch_wgrad(const uint8_t* ac, const uint8_t* as, const uint8_t* bc, const uint8_t* bs,
                         const int32_t* off, int E, int64_t N1, int64_t N2, float* dw, float beta, bool zero_empty,
                         hipStream_t s) {
  const XcdSplit xs = xcd_split((N1 + wsg2::TM - 1) / wsg2::TM, (N2 + wsg2::TN - 1) / wsg2::TN, wsg2::TM, wsg2::TN);
  const int64_t ws2_all = 8ll * xs.pm * xs.pn * E;
  if (E <= wsg::MAX_E && ws2_all < (1ll << 31) && (int64_t)N1 * N2 * 4 < (1ll << 31)) {
    int64_t grid = cu_count();
    if (grid > ws2_all) grid = ws2_all;
    hipLaunchKernelGGL(k_wgrad_ws256, dim3((unsigned)grid), dim3(wsg::NT), 0, s, ac, as, bc, bs, off, E, N1, N2, xs,
                       ws2_all, dw, beta, zero_empty);
    return;
  }
  const int64_t ws_all = (N2 + wsg::TN - 1) / wsg::TN * ((N1 + wsg::TM - 1) / wsg::TM) * E;
  if (E <= wsg::MAX_E && ws_all < (1ll << 31) && (int64_t)N1 * N2 * 4 < (1ll << 31)) {
    const int64_t n_nt = (N2 + wsg::TN - 1) / wsg::TN;
    int64_t grid = cu_count();
    if (grid > ws_all) grid = ws_all;
    hipLaunchKernelGGL(k_wgrad_ws, dim3((unsigned)grid), dim3(wsg::NT), 0, s, ac, as, bc, bs, off, E, N1, N2, n_nt,
                       ws_all, dw, beta, zero_empty);
    return;
  }
  launch_wgrad_t<128, 128, 2, 2, 2>(ac, as, bc, bs, off, E, N1, N2, dw, beta, zero_empty, s);
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
  MOE4_REQUIRE(M_total * K < ((int64_t)1 << 31) && N * K < ((int64_t)1 << 31), MOE4_EINVAL,
               "moe_grouped_gemm_bwd_dgrad: A and each expert's B must stay below 2 GiB");
  if (M_total == 0) return MOE4_OK;
  launch_dgrad(a_codes, a_sf, b_codes, b_sf, expert_off, E, M_total, N, K, c, as_stream(stream));
  return check_launch("moe_grouped_gemm_bwd_dgrad");
}

extern "C" int moe_grouped_gemm_mx(const uint8_t* a_codes, const uint8_t* a_sf, const uint8_t* b_codes,
                                   const uint8_t* b_sf, const int32_t* expert_off, int32_t E, int64_t M_total,
                                   int64_t N, int64_t K, void* c, int c_dtype, void* stream) {
  MOE4_REQUIRE(c_dtype == MOE4_F32 || c_dtype == MOE4_BF16, MOE4_EINVAL, "moe_grouped_gemm_mx: c_dtype must be F32 or BF16");
  if (c_dtype == MOE4_F32)
    return moe_grouped_gemm_bwd_dgrad(a_codes, a_sf, b_codes, b_sf, expert_off, E, M_total, N, K, static_cast<float*>(c),
                                      stream);
  MOE4_REQUIRE(E >= 1 && M_total >= 0 && N > 0 && K > 0 && K % dmag::BK == 0 && N % 32 == 0, MOE4_EINVAL,
               "moe_grouped_gemm_mx: bf16 output needs K % 128 == 0 and N % 32 == 0");
  MOE4_REQUIRE(b_codes && b_sf && expert_off, MOE4_EINVAL, "moe_grouped_gemm_mx: NULL pointer");
  MOE4_REQUIRE(M_total == 0 || (a_codes && a_sf && c), MOE4_EINVAL, "moe_grouped_gemm_mx: NULL pointer");
  MOE4_REQUIRE(aligned16(a_codes) && aligned16(b_codes) && aligned16(c), MOE4_EALIGN,
               "moe_grouped_gemm_mx: misaligned pointer");
  MOE4_REQUIRE(M_total * K < ((int64_t)1 << 31) && N * K < ((int64_t)1 << 31), MOE4_EINVAL,
               "moe_grouped_gemm_mx: A and each expert's B must stay below 2 GiB");
  if (M_total == 0) return MOE4_OK;
  if (N % 128 == 0) {
    if (N % 256 == 0)
      hipLaunchKernelGGL((k_dgrad_ws<true, 256>), dim3((unsigned)(cu_count() < 8 ? 8 : cu_count())), dim3(dws::NT), 0, as_stream(stream),
                         a_codes, a_sf, b_codes, b_sf, expert_off, E, M_total, N, K, dg_split(N / 256, dws::TM, 256), c);
    else
      hipLaunchKernelGGL((k_dgrad_ws<true, 128>), dim3((unsigned)(cu_count() < 8 ? 8 : cu_count())), dim3(dws::NT), 0, as_stream(stream),
                         a_codes, a_sf, b_codes, b_sf, expert_off, E, M_total, N, K, dg_split(N / 128, dws::TM, 128), c);
    return check_launch("moe_grouped_gemm_mx");
  }
  const int64_t n_nt = (N + 255) / 256;
  const int64_t n_all = n_nt * ((M_total + 255) / 256 + E);
  hipLaunchKernelGGL(k_mx_gemm_dma_256_bf16, dim3((unsigned)xcd_grid(n_all)), dim3(dmag::NT), 0, as_stream(stream),
                     a_codes, a_sf, b_codes, b_sf, expert_off, E, M_total, N, K, n_nt, n_all, c);
  return check_launch("moe_grouped_gemm_mx");
}

extern "C" int moe_grouped_gemm_bwd_wgrad(const uint8_t* a_codes, const uint8_t* a_sf, const uint8_t* b_codes,
                                          const uint8_t* b_sf, const int32_t* expert_off_pad, int32_t E, int64_t N1,
                                          int64_t N2, float* dw, float beta, int flags, void* stream) {
  MOE4_REQUIRE(E >= 1 && N1 > 0 && N2 > 0 && N1 % 32 == 0 && N2 % 32 == 0, MOE4_EINVAL,
               "moe_grouped_gemm_bwd_wgrad: need N1 % 32 == 0 and N2 % 32 == 0");
  MOE4_REQUIRE(beta == 0.0f || beta == 1.0f, MOE4_EINVAL, "moe_grouped_gemm_bwd_wgrad: beta must be 0 or 1");
  MOE4_REQUIRE((flags & ~MOE4_WGRAD_SKIP_EMPTY) == 0, MOE4_EINVAL, "moe_grouped_gemm_bwd_wgrad: unknown flags");
  MOE4_REQUIRE(a_codes && a_sf && b_codes && b_sf && expert_off_pad && dw, MOE4_EINVAL,
               "moe_grouped_gemm_bwd_wgrad: NULL pointer");
  MOE4_REQUIRE(aligned16(a_codes) && aligned16(b_codes) && aligned16(dw), MOE4_EALIGN,
               "moe_grouped_gemm_bwd_wgrad: misaligned pointer");
  MOE4_REQUIRE(((N2 + 127) / 128) * ((N1 + 127) / 128) * E < ((int64_t)1 << 31), MOE4_EINVAL,
               "moe_grouped_gemm_bwd_wgrad: too large");
  launch_wgrad(a_codes, a_sf, b_codes, b_sf, expert_off_pad, E, N1, N2, dw, beta, (flags & MOE4_WGRAD_SKIP_EMPTY) == 0,
               as_stream(stream));
  return check_launch("moe_grouped_gemm_bwd_wgrad");
}

extern "C" int moe_grouped_gemm_bwd(const uint8_t* dy_codes, const uint8_t* dy_sf, const uint8_t* wT_codes,
                                    const uint8_t* wT_sf, const uint8_t* dyT_codes, const uint8_t* dyT_sf,
                                    const uint8_t* xT_codes, const uint8_t* xT_sf, const int32_t* expert_off,
                                    const int32_t* expert_off_pad, int32_t E, int64_t M_total, int64_t Nin,
                                    int64_t Nout, float* dx, float* dw, float beta, int flags, void* stream) {
  int rc = moe_grouped_gemm_bwd_dgrad(dy_codes, dy_sf, wT_codes, wT_sf, expert_off, E, M_total, Nin, Nout, dx, stream);
  if (rc) return rc;
  return moe_grouped_gemm_bwd_wgrad(dyT_codes, dyT_sf, xT_codes, xT_sf, expert_off_pad, E, Nout, Nin, dw, beta, flags,
                                    stream);
}
