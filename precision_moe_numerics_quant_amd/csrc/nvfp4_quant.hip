// NVFP4 quantisation with the Four-Over-Six block-scale choice (gfx950).
//
// Two-level scaling as the lhc.media page describes NVFP4 (4-bit values plus
// a scale per sixteen values) with a float32 tensor scale per row group, and
// the 4/6 choice of the agihunt.info page, "Confirmed": per 16-block keep the
// candidate (block amax mapped to 6, or to 4) with the lower squared error.
//
// Kernels, in launch order:
//   k_zero_u32      clear the per-group amax words (workspace)
//   k_amax          per-group max |x| (float bits, atomicMax: order-free);
//                   persistent coalesced walk
//   k_tensor_scale  S_g = fl(amax_g / (m_max * 448)), 1 for a zero group
//   k_encode        one thread per 16-element block: both candidates, errors
//                   in the fixed order, the choice, packed codes + scale byte
// and, for weights, k_encode_requant_T in place of all three: the group amax,
// the mode-6 codes and, from them, the stochastic-rounding transposed MXFP8
// copy the backward pass needs, in one persistent launch.
// All float arithmetic is one IEEE binary32 operation per step (the library
// is built with -ffp-contract=off), with correctly rounded division.
#include <mutex>
#include <string>
#include <type_traits>

#include "act.h"
#include "gemm_common.h"
#include "moe4_internal.h"
#include "mx_requant.h"
#include "nvfp4_enc.h"

namespace moe4 {

__global__ void k_zero_u32(uint32_t* p, int n) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// Group of row r for offsets off[0..G] (largest g with off[g] <= r).
__device__ inline int group_of_row(const int32_t* off, int G, int64_t r) {
  if (off == nullptr) return 0;
  int lo = 0, hi = G - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if ((int64_t)off[mid] <= r) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Load 8 consecutive source values of row-major x as float32 (applying SiLU).
template <int DT, bool SILU>
__device__ inline void load8(const void* x, int64_t idx, float* v, const float* tab) {
  if (DT == MOE4_BF16) {
    u32x4 w = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(x) + idx);
    if (SILU) {
      const uint32_t ww[4] = {w[0], w[1], w[2], w[3]};
      float t[8];
      act_eval_packed<false>(ww, tab, t);
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = t[i];
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] = bf16_bits_to_f32(w[i] & 0xFFFFu);
        v[2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
      }
    }
  } else {
    const f32x4* p = reinterpret_cast<const f32x4*>(static_cast<const float*>(x) + idx);
    f32x4 a = p[0], b = p[1];
#pragma unroll
    for (int i = 0; i < 4; ++i) { v[i] = a[i]; v[4 + i] = b[i]; }
  }
}

// ------------------------------------------------------------ chunk walk
// Both passes walk the flat row-major tensor in chunks of 1024 elements; each
// wave of the persistent grid owns a contiguous run of chunks and keeps the
// next chunk's loads in flight while it works on the current one.  Lane l reads
// the 16-byte pieces k*64 + l (k < NLD) of its chunk, so every load
// instruction covers 1 KB contiguously; a piece holds EPL elements and a
// 16-element block spans LPB = 16 / EPL adjacent lanes.
template <int DT>
struct Walk {
  static constexpr int EPL = DT == MOE4_F32 ? 4 : 8;
  static constexpr int NLD = 16 / EPL;
  static constexpr int LPB = 16 / EPL;
  static constexpr int CHUNK = 1024;
};

// EPL source values of piece index p (element p * EPL) as float32, SiLU applied.
template <int DT, bool SILU>
__device__ inline void load_piece(const void* x, int64_t p, float (&v)[Walk<DT>::EPL], const float* tab) {
  if (DT == MOE4_F32) {
    f32x4 a = reinterpret_cast<const f32x4*>(x)[p];
    v[0] = a[0]; v[1] = a[1]; v[2] = a[2]; v[3] = a[3];
  } else {
    u32x4 w = reinterpret_cast<const u32x4*>(x)[p];
    if constexpr (SILU) {
      const uint32_t ww[4] = {w[0], w[1], w[2], w[3]};
      act_eval_packed<false>(ww, tab, v);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] = bf16_bits_to_f32(w[i] & 0xFFFFu);
        v[2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
      }
    }
  }
}

// Group of row r, searching forward from g (rows only grow along a wave's walk).
__device__ inline int group_from(const int32_t* off, int G, int g, int64_t r) {
  while (g + 1 < G && (int64_t)off[g + 1] <= r) ++g;
  return g;
}

// A wave's walk: the contiguous chunk range [c, c_end) (block distribution,
// so group boundaries are met rarely), the group gw of the current rows and
// the row where it ends (cached: the common chunk needs no offset loads).
struct WaveWalk {
  int64_t c, c_end;
  int gw;
  int64_t g_end;
  int64_t ge_elem;  // g_end * cols (the first element past group gw)
  __device__ void init(int64_t n_chunks, int chunk, int64_t cols, const int32_t* goff, int G) {
    const int64_t wave = (int64_t)blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);
    const int64_t n_waves = (int64_t)gridDim.x * (blockDim.x / 64);
    const int64_t per = (n_chunks + n_waves - 1) / n_waves;
    c = wave * per;
    c_end = c + per < n_chunks ? c + per : n_chunks;
    gw = 0;
    g_end = INT64_MAX;
    ge_elem = INT64_MAX;
    if (goff && c < c_end) {
      gw = group_of_row(goff, G, c * chunk / cols);
      g_end = gw + 1 < G ? (int64_t)goff[gw + 1] : INT64_MAX;
      ge_elem = g_end == INT64_MAX ? INT64_MAX : g_end * cols;
    }
  }
  // move gw forward to the group of row r
  __device__ void advance(const int32_t* goff, int G, int64_t r, int64_t cols) {
    if (r < g_end) return;
    gw = group_from(goff, G, gw, r);
    g_end = gw + 1 < G ? (int64_t)goff[gw + 1] : INT64_MAX;
    ge_elem = g_end == INT64_MAX ? INT64_MAX : g_end * cols;
  }
};

constexpr int QTHREADS = 256;

// Group maxima of the amax walk: each group has `slots` words, and workgroup
// b folds into word b % slots of its group, so that a tensor of one group
// (thousands of workgroups) does not serialise all its atomics on one word.
__host__ __device__ inline int amax_slots(int G) { return G <= 512 ? 8 : 1; }

// End of a walk: the workgroup's waves combine their maxima of the same group
// in LDS, then one atomic maximum per distinct group (waves walk consecutive
// chunk ranges, so the groups come in ascending order).
__device__ inline void amax_flush_wg(int gw, float t, bool has, uint32_t* amax_bits, int slots) {
  __shared__ int s_g[QTHREADS / 64];
  __shared__ float s_t[QTHREADS / 64];
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    s_g[w] = has ? gw : -1;
    s_t[w] = t;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t slot = blockIdx.x % (uint32_t)slots;
    int g = -1;
    float m = 0.0f;
    for (int k = 0; k < QTHREADS / 64; ++k) {
      if (s_g[k] < 0) continue;
      if (s_g[k] != g) {
        if (g >= 0) atomicMax(amax_bits + (size_t)g * slots + slot, __float_as_uint(m));
        g = s_g[k];
        m = 0.0f;
      }
      m = fmaxf(m, s_t[k]);
    }
    if (g >= 0) atomicMax(amax_bits + (size_t)g * slots + slot, __float_as_uint(m));  // m >= 0: bit order = value order
  }
}

template <int DT, bool SILU>
__global__ void __launch_bounds__(QTHREADS) k_amax(const void* __restrict__ x, int64_t rows, int64_t cols,
                                                   const int32_t* __restrict__ goff, int G,
                                                   uint32_t* __restrict__ amax_bits,
                                                   const float* __restrict__ act_tab, int slots) {
  using W = Walk<DT>;
  const uint32_t slot = blockIdx.x % (uint32_t)slots;
  static_assert(!SILU || DT == MOE4_BF16, "SiLU applies to bf16 sources");
  const int64_t n = rows * cols, n_chunks = (n + W::CHUNK - 1) / W::CHUNK;
  const int l = threadIdx.x & 63;
  WaveWalk ww;
  ww.init(n_chunks, W::CHUNK, cols, goff, G);
  if constexpr (SILU) {
    // max |silu(u)| over bf16 u without evaluating silu per element.  The
    // correctly rounded silu is non-decreasing on [0, inf); |silu| is
    // non-decreasing in u on (-inf, u*] and non-increasing on [u*, 0), u* ~
    // -1.2785 the minimum of silu; rounding keeps monotonicity, and the
    // adjacent bf16 values -1.28125 < u* < -1.2734375 split the negatives into
    // those two ranges.  So the maximum is the largest of silu(largest u >= 0),
    // |silu(largest u <= -1.28125)| and |silu(smallest u in [-1.2734375, 0))|:
    // three integer extremes of the bit patterns per lane, and three table
    // reads per flush.
    constexpr uint32_t M1 = 0x3FA4u;  // |-1.28125| in bf16; 0x3FA3 is |-1.2734375|
    uint32_t pmax = 0u, nlo = 0x8000u, nhi = 0u;  // (0x8000: no value <= -1.28125 yet)
    float mf = 0.0f;                              // pieces folded directly (group boundaries)
    auto fold = [&](uint32_t b) {
      const uint32_t m = b & 0x7FFFu;
      const bool neg = b >= 0x8000u;
      pmax = max(pmax, neg ? 0u : m);
      nlo = min(nlo, neg && m >= M1 ? m : 0x8000u);
      nhi = max(nhi, neg && m < M1 ? m : 0u);
    };
    auto lane_amax = [&]() {
      float t = fmaxf(mf, act_eval<false>(pmax, act_tab));
      if (nlo < 0x8000u) t = fmaxf(t, fabsf(act_eval<false>(0x8000u | nlo, act_tab)));
      return fmaxf(t, fabsf(act_eval<false>(0x8000u | nhi, act_tab)));
    };
    auto load_raw = [&](int64_t c, u32x4 (&w)[W::NLD]) {
#pragma unroll
      for (int k = 0; k < W::NLD; ++k) {
        const int64_t p = c * (W::CHUNK / W::EPL) + k * 64 + l;
        w[k] = (c < ww.c_end && p * W::EPL < n) ? reinterpret_cast<const u32x4*>(x)[p] : u32x4{0u, 0u, 0u, 0u};
      }
    };
    u32x4 w[W::NLD], wn[W::NLD];
    load_raw(ww.c, w);
    for (int64_t c = ww.c; c < ww.c_end; ++c) {
      load_raw(c + 1, wn);
      const int64_t e0 = c * W::CHUNK;
      const int64_t e_end = e0 + W::CHUNK < n ? e0 + W::CHUNK : n;
      if (e_end <= ww.ge_elem) {  // the chunk stays in group gw (no division on the common path)
#pragma unroll
        for (int k = 0; k < W::NLD; ++k)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            fold(w[k][i] & 0xFFFFu);
            fold(w[k][i] >> 16);
          }
      } else {  // the chunk reaches past group gw: per-piece groups, then move on
#pragma unroll
        for (int k = 0; k < W::NLD; ++k) {
          const int64_t e = e0 + (int64_t)(k * 64 + l) * W::EPL;
          if (e < n) {
            float t = 0.0f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              t = fmaxf(t, fabsf(act_eval<false>(w[k][i] & 0xFFFFu, act_tab)));
              t = fmaxf(t, fabsf(act_eval<false>(w[k][i] >> 16, act_tab)));
            }
            const int gp = group_from(goff, G, ww.gw, e / cols);
            if (gp == ww.gw) mf = fmaxf(mf, t);
            else atomicMax(amax_bits + (size_t)gp * slots + slot, __float_as_uint(t));
          }
        }
        const float t = wave_max(lane_amax());
        if (l == 0) atomicMax(amax_bits + (size_t)ww.gw * slots + slot, __float_as_uint(t));
        pmax = 0u;
        nlo = 0x8000u;
        nhi = 0u;
        mf = 0.0f;
        ww.advance(goff, G, (e_end - 1) / cols, cols);
      }
#pragma unroll
      for (int k = 0; k < W::NLD; ++k) w[k] = wn[k];
    }
    amax_flush_wg(ww.gw, wave_max(lane_amax()), ww.c < ww.c_end, amax_bits, slots);
    return;
  }
  const float* tab = act_tab;  // (unused without SiLU)
  float m = 0.0f;  // this lane's running maximum of group ww.gw
  auto load_chunk = [&](int64_t c, float (&v)[W::NLD][W::EPL]) {
#pragma unroll
    for (int k = 0; k < W::NLD; ++k) {
      const int64_t p = c * (W::CHUNK / W::EPL) + k * 64 + l;
      if (c < ww.c_end && p * W::EPL < n) load_piece<DT, SILU>(x, p, v[k], tab);
      else
#pragma unroll
        for (int i = 0; i < W::EPL; ++i) v[k][i] = 0.0f;
    }
  };
  float v[W::NLD][W::EPL], vn[W::NLD][W::EPL];
  load_chunk(ww.c, v);
  for (int64_t c = ww.c; c < ww.c_end; ++c) {
    load_chunk(c + 1, vn);  // next chunk in flight while this one is reduced
    const int64_t e0 = c * W::CHUNK;
    const int64_t e_end = e0 + W::CHUNK < n ? e0 + W::CHUNK : n;
    if (e_end <= ww.ge_elem) {  // the chunk stays in group gw (no division on the common path)
#pragma unroll
      for (int k = 0; k < W::NLD; ++k)
#pragma unroll
        for (int i = 0; i < W::EPL; ++i) m = fmaxf(m, fabsf(v[k][i]));
    } else {  // the chunk reaches past group gw: per-piece groups, then move on
#pragma unroll
      for (int k = 0; k < W::NLD; ++k) {
        const int64_t e = e0 + (int64_t)(k * 64 + l) * W::EPL;
        if (e < n) {
          float t = 0.0f;
#pragma unroll
          for (int i = 0; i < W::EPL; ++i) t = fmaxf(t, fabsf(v[k][i]));
          const int gp = group_from(goff, G, ww.gw, e / cols);
          if (gp == ww.gw) m = fmaxf(m, t);
          else atomicMax(amax_bits + (size_t)gp * slots + slot, __float_as_uint(t));
        }
      }
      const float t = wave_max(m);
      if (l == 0) atomicMax(amax_bits + (size_t)ww.gw * slots + slot, __float_as_uint(t));
      m = 0.0f;
      ww.advance(goff, G, (e_end - 1) / cols, cols);
    }
#pragma unroll
    for (int k = 0; k < W::NLD; ++k)
#pragma unroll
      for (int i = 0; i < W::EPL; ++i) v[k][i] = vn[k][i];
  }
  amax_flush_wg(ww.gw, wave_max(m), ww.c < ww.c_end, amax_bits, slots);
}

__global__ void k_tensor_scale(const uint32_t* __restrict__ amax_bits, int G, float m_max448,
                               float* __restrict__ ts, int slots = 1) {
  int g = blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= G) return;
  uint32_t b = 0u;
  for (int k = 0; k < slots; ++k) b = max(b, amax_bits[(size_t)g * slots + k]);
  float s = __uint_as_float(b) / m_max448;
  ts[g] = (s == 0.0f) ? 1.0f : s;
}

constexpr int ENC_THREADS = 256;

template <int DT, bool SILU, bool FOUR_OVER_SIX>
__global__ void __launch_bounds__(ENC_THREADS) k_encode(const void* __restrict__ x, int64_t rows, int64_t cols,
                                                        const int32_t* __restrict__ goff, int G,
                                                        const float* __restrict__ ts,
                                                        uint8_t* __restrict__ codes, uint8_t* __restrict__ sf,
                                                        const float* __restrict__ act_tab, int bpt) {
  __shared__ float tab[SILU ? ACT_TAB : 1];
  if (SILU) stage_act_table(tab, act_tab);
  const int64_t nbr = cols / 16;
  // bpt blocks per thread (SiLU: amortises the table staging)
  for (int it = 0; it < bpt; ++it) {
  const int64_t blk0 = ((int64_t)blockIdx.x * bpt + it) * ENC_THREADS + (threadIdx.x & ~63);  // the wave's first block
  const int64_t blk = blk0 + (threadIdx.x & 63);
  if (blk >= rows * nbr) return;
  int g = 0;
  if (goff != nullptr) {
    // group of the row: the wave's first row by one scalar division and one
    // search (uniform: scalar loads), the lane's row by stepping from there
    const int64_t bw = (int64_t)__builtin_amdgcn_readfirstlane((int)(blk0 & 0x7FFFFFFF)) |
                       ((int64_t)__builtin_amdgcn_readfirstlane((int)(blk0 >> 31)) << 31);
    const int64_t r_wave = bw / nbr;
    int64_t r = r_wave, rem = bw - r_wave * nbr + (threadIdx.x & 63);
    while (rem >= nbr) {
      rem -= nbr;
      ++r;
    }
    g = __builtin_amdgcn_readfirstlane(group_of_row(goff, G, r_wave));
    if (g + 1 < G && (int64_t)goff[g + 1] <= r)  // (goff[g + 1]: a scalar load)
      while (g + 1 < G && (int64_t)goff[g + 1] <= r) ++g;
  }
  const float S = ts[g];
  float v[16];
  load8<DT, SILU>(x, blk * 16, v, tab);
  load8<DT, SILU>(x, blk * 16 + 8, v + 8, tab);
  float amax_b = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax_b = fmaxf(amax_b, fabsf(v[i]));
  // the common case without the zero-scale and infinite-reciprocal branches;
  // a wave with a lane in either case redoes both candidates with them
  bool ok6 = true, ok4 = true;
  Cand best = encode_candidate_fast(v, amax_b, S, 6.0f, ok6);
  Cand c4;
  if (FOUR_OVER_SIX) c4 = encode_candidate_fast(v, amax_b, S, 4.0f, ok4);
  if (__builtin_expect(__any(!(ok6 && ok4)), 0)) {
    best = encode_candidate(v, amax_b, S, 6.0f);
    if (FOUR_OVER_SIX) c4 = encode_candidate(v, amax_b, S, 4.0f);
  }
  if (FOUR_OVER_SIX && c4.err < best.err) best = c4;
  *reinterpret_cast<u32x2*>(codes + blk * 8) = u32x2{best.q[0], best.q[1]};
  sf[blk] = (uint8_t)best.sc;
  }
}

static int cu_count_q() {
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

// Persistent grid: enough 1024-element wave chunks, at most 8 workgroups per CU.
static dim3 walk_grid(int64_t n) {
  const int64_t waves = (n + 1023) / 1024;
  int64_t wg = (waves + QTHREADS / 64 - 1) / (QTHREADS / 64);
  const int64_t cap = (int64_t)cu_count_q() * 8;
  if (wg > cap) wg = cap;
  if (wg < 1) wg = 1;
  return dim3((unsigned)wg);
}

template <int DT, bool SILU>
static void launch_encode(bool four6, dim3 grid, hipStream_t s, const void* x, int64_t rows, int64_t cols,
                          const int32_t* goff, int G, const float* ts, uint8_t* codes, uint8_t* sf,
                          const float* tab) {
  const int bpt = SILU ? 16 : 1;
  grid.x = (unsigned)((rows * (cols / 16) + (int64_t)ENC_THREADS * bpt - 1) / ((int64_t)ENC_THREADS * bpt));
  if (four6)
    hipLaunchKernelGGL((k_encode<DT, SILU, true>), grid, dim3(ENC_THREADS), 0, s, x, rows, cols, goff, G, ts,
                       codes, sf, tab, bpt);
  else
    hipLaunchKernelGGL((k_encode<DT, SILU, false>), grid, dim3(ENC_THREADS), 0, s, x, rows, cols, goff, G, ts,
                       codes, sf, tab, bpt);
}

// Weights, fused: float32 [G * grows, C] -> NVFP4 mode 6 (codes, scales and
// the per-group tensor scales) and, from the same codes and the same steps as
// k_requant_T, the transposed MXFP8 stochastic-rounding copy (group-major,
// grows rows per group, no padding, row-major scales), in one persistent
// launch.  Tile: 4 waves x (32 rows = one MX block) x 512 columns of one
// group; lane l of wave w takes columns c0 + 8l .. c0 + 8l + 7 of the wave's
// 32 rows, so lanes 2m and 2m+1 hold one 16-element NVFP4 block (its amax
// through one shuffle) and each lane keeps its 32 code words for the
// requantisation.
//
// The group amax must be complete before any of the group's blocks is
// encoded, so the launch walks the tiles twice, taking tickets from a counter
// in the workspace: tickets 0 .. n-1 fold tile t into its group's amax,
// tickets n .. 2n-1 encode tile t - n after waiting for the group's amax
// count.  Every tile of that group has a lower ticket, taken by a workgroup
// that is running and never waits during an amax: the wait always ends (and
// is bounded anyway; a give-up sets MOE4_DEVERR_WAIT in this file's device
// error word, which moe4_debug_check reports).  One launch
// instead of amax, tensor-scale and encode kernels removes two launch tails.
// (Pairing each amax with an encode a few groups behind, so that the encode's
// re-read hits the memory-side cache, measured slower: the encode is bound by
// its ALU work and load latency at two workgroups per CU, not by HBM.)
namespace wq {
constexpr uint32_t SPIN_LIMIT = 1u << 22;
constexpr uint32_t FORCED_SPIN_LIMIT = 64;  // moe4_debug_force_wait_timeout
}

// This file's device-side error word (moe4_debug_check reads and clears it).
static __device__ uint32_t g_dev_err;
uint32_t take_dev_err_nvfp4() { return take_device_word(&g_dev_err); }

__global__ void __launch_bounds__(rq::THREADS) __attribute__((amdgpu_waves_per_eu(2, 2))) k_encode_requant_T(const float* __restrict__ x, int64_t C,
                                                                  int64_t grows, int G, uint32_t n_ct,
                                                                  uint32_t n_item, uint32_t wait_extra, uint32_t spin_limit,
                                                                  uint32_t* __restrict__ wsu, float* __restrict__ ts,
                                                                  uint32_t base, uint8_t* __restrict__ codes,
                                                                  uint8_t* __restrict__ sf, uint8_t* __restrict__ out_c,
                                                                  uint8_t* __restrict__ out_s) {
  using namespace rq;
  __shared__ __attribute__((aligned(16))) uint8_t lq[COLS * ROWS];
  __shared__ uint8_t lsf[COLS * WAVES];  // [column][block]
  __shared__ int64_t lblk[WAVES][3];
  __shared__ float s_red[WAVES];
  __shared__ float s_S;
  __shared__ uint32_t s_tk;
  // Per group the float bits of the amax so far and the number of amax tiles
  // folded in.  Device-scope atomics are performed at the memory side, so the
  // two words need no cache fences, only order: the count is bumped after the
  // maximum has returned, and read before the maximum.
  uint32_t* amax = wsu;      // [G]
  uint32_t* done = wsu + G;  // [G]
  uint32_t* ticket = wsu + 2 * G;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const uint32_t n_all = (uint32_t)G * n_item, n_tk = 2 * n_all;
  const uint32_t key0 = fmix32(base);
  if (tid == 0) s_tk = atomicAdd(ticket, 1u);
  __syncthreads();
  uint32_t t = __builtin_amdgcn_readfirstlane(s_tk);
  while (t < n_tk) {
    uint32_t t_next = 0;
    if (tid == 0) t_next = atomicAdd(ticket, 1u);  // in flight during this ticket
    if (t < n_all) {  // ---- amax of tile t
      const uint32_t g = t / n_item, j = t - g * n_item, jr = j / n_ct;
      const int64_t pr = (int64_t)jr * ROWS + 32 * w, c = (int64_t)(j - jr * n_ct) * COLS + LCOLS * l;
      float m = 0.0f;
      if (pr < grows && c < C) {
        const float* xr = x + ((int64_t)g * grows + pr) * C + c;
        f32x4 vb[2][4][2];
        auto load4 = [&](int k, f32x4 (&b)[4][2]) {
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) {
            const f32x4* q = reinterpret_cast<const f32x4*>(xr + (int64_t)(4 * k + ii) * C);
            b[ii][0] = q[0];
            b[ii][1] = q[1];
          }
        };
        load4(0, vb[0]);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          if (k + 1 < 8) load4(k + 1, vb[(k + 1) & 1]);
#pragma unroll
          for (int ii = 0; ii < 4; ++ii)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              m = fmaxf(m, fmaxf(fabsf(vb[k & 1][ii][0][e]), fabsf(vb[k & 1][ii][1][e])));
        }
      }
      m = wave_max(m);
      if (l == 0) s_red[w] = m;
      __syncthreads();
      if (tid == 0) {
        float mm = s_red[0];
#pragma unroll
        for (int q = 1; q < WAVES; ++q) mm = fmaxf(mm, s_red[q]);
        // mm >= 0: its bit pattern orders as its value, and the old value's
        // sign bit (always 0) makes the count wait for the maximum's return
        const uint32_t old = __hip_atomic_fetch_max(amax + g, __float_as_uint(mm), __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_fetch_add(done + g, 1u + (old >> 31), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    else {  // ---- encode + requantise tile t - n_all
      const uint32_t it = t - n_all, g = it / n_item, j = it - g * n_item, jr = j / n_ct;
      const int64_t c0 = (int64_t)(j - jr * n_ct) * COLS, pr = (int64_t)jr * ROWS + 32 * w;  // wave's first row in g
      const bool present = pr < grows;
      const int64_t r0 = (int64_t)g * grows + pr;
      if (tid == 0) {
        // (wait_extra is 0; the test hook sets it to 1, a count that never
        // arrives, with a tiny spin_limit)
        uint32_t n = 0, spins = 0;
        while ((n = __hip_atomic_load(done + g, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) < n_item + wait_extra &&
               ++spins < spin_limit)
          __builtin_amdgcn_s_sleep(8);
        if (n < n_item + wait_extra) atomicOr(&g_dev_err, MOE4_DEVERR_WAIT);
        // (n >> 31 is 0: the address waits for the count)
        const float a = __uint_as_float(__hip_atomic_load(amax + g + (n >> 31), __ATOMIC_RELAXED,
                                                          __HIP_MEMORY_SCOPE_AGENT));
        const float sv = a / (6.0f * 448.0f);
        s_S = (sv == 0.0f) ? 1.0f : sv;
        if (j == 0) ts[g] = s_S;
      }
      if (l == 0) {
        lblk[w][0] = C * (int64_t)g * grows + pr;
        lblk[w][1] = present ? grows : 0;
        lblk[w][2] = C * (int64_t)g * grows / 32 + pr / 32;
      }
      __syncthreads();
      const float S = s_S;
      const int64_t c = c0 + LCOLS * l;
      auto put = [&](int k, int q, uint32_t v) {
        const int col = LCOLS * l + q;
        *reinterpret_cast<uint32_t*>(lq + col * ROWS + swz(col, 2 * w + (k >> 2)) * 16 + (k & 3) * 4) = v;
      };
      int ex[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) ex[q] = -127;
      if (present && c < C) {  // (C % 16 == 0: both lanes of a 16-block agree)
        const float* xr = x + r0 * C + c;
        uint32_t cw[32], sbp[8];
        float am[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) sbp[k] = 0u;
#pragma unroll
        for (int q = 0; q < 8; ++q) am[q] = 0.0f;
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
            a = fmaxf(a, __shfl_xor(a, 1, 64));  // the block's other half
            uint32_t sc;
            cw[i] = encode_half(v, a, S, 6.0f, sc);
            sbp[k] |= sc << (8 * ii);
            *reinterpret_cast<uint32_t*>(codes + (r0 + i) * (C / 2) + c / 2) = cw[i];
            if ((l & 1) == 0) sf[(r0 + i) * (C / 16) + c / 16] = (uint8_t)sc;
            float q8[8];
            dequant8(cw[i], sc, q8);
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
        // decode again below instead of keeping the 256 decoded values live
#pragma unroll
        for (int i = 0; i < 32; ++i) asm volatile("" : "+v"(cw[i]));
        const int64_t j0 = r0 * (C / 2) + c / 2;  // pair index of (row r0, column c)
        auto deq = [&](int i, float (&q)[8]) { dequant8(cw[i], (sbp[i >> 2] >> (8 * (i & 3))) & 0xFFu, q); };
        const bool fast = j0 + 31 * (C / 2) + 3 < ((int64_t)1 << 32);
        if (fold_scale_ok(S)) {  // one multiply by S * 2^-ex per value (the same values)
          float f[8];
#pragma unroll
          for (int q = 0; q < 8; ++q) f[q] = ex[q] == -127 ? 0.0f : S * pc[q];
          if (fast) requant_block<true, true>(deq, 32, 1.0f, f, j0, C / 2, base, key0, put);
          else requant_block<false, true>(deq, 32, 1.0f, f, j0, C / 2, base, key0, put);
        } else if (fast) {
          requant_block<true, true>(deq, 32, S, pc, j0, C / 2, base, key0, put);
        } else {
          requant_block<false, true>(deq, 32, S, pc, j0, C / 2, base, key0, put);
        }
      } else {
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
    __syncthreads();  // LDS free for the next ticket
    if (tid == 0) s_tk = t_next;
    __syncthreads();
    t = __builtin_amdgcn_readfirstlane(s_tk);
  }
}

// Weights, fused, one HBM read: the same outputs as k_encode_requant_T for
// groups whose tiles all fit the chip at once.  Each workgroup owns one
// 32-row x 256-column tile (rows of 1 KB), the same one in every group (G
// rounds), and holds its float32 values in registers from the amax to the
// encode: lane l of wave w takes rows 4 (l / 8) .. + 3 and columns
// 64 w + 8 (l % 8) .. + 7 of the tile, so a 16-value NVFP4 block lies in the
// lanes l, l ^ 1 and a 32-row MX block in the lanes l, l ^ 8, l ^ 16, l ^ 32.
// Four register sets rotate: in round g the workgroup folds group g + 2's
// tile into its maximum and publishes it, encodes group g (whose tensor
// scale it took at the end of the previous round) and stores it, takes group
// g + 1's tensor scale (every workgroup published its part a round earlier,
// so the wait normally finds it complete) and issues group g + 4's loads into
// the freed set.  Wave 0 publishes and polls and does no global store (its
// polls would queue behind the stores, a wave's memory operations
// completing in order), and loads after its poll; waves 1-3 write the tile's
// outputs from LDS in 16-byte pieces.  Tiles are numbered so that the four
// tiles of a 128-row run sit on one XCD (workgroup b runs on XCD b % 8),
// whose L2 then merges their 32-byte pieces of each MXFP8 column.  The
// launch needs every workgroup resident (checked against the occupancy on
// the host); the wait is bounded like k_encode_requant_T's and a give-up sets
// MOE4_DEVERR_WAIT.
namespace wr {
constexpr int WAVES = 4, THREADS = 64 * WAVES, TR = 32, TC = 256, MIN_BLOCKS = 3;
// Group maxima without atomics: workgroup b stores its tile's maximum, its
// top bit set as a presence mark (the bits of a maximum, a non-negative
// float, have it clear), into word b of the group's n_tile workspace words;
// every workgroup reads all of them back (wave 0, 12 words per lane) until
// all are present, and takes the same maximum and tensor scale.  A chain of
// one store and one read per group (returning atomics, chained, cost several
// memory round trips each, and hundreds of them on one word serialise).
constexpr int MAX_TILES = 768;
}

template <bool FAST>
__global__ void __launch_bounds__(wr::THREADS, wr::MIN_BLOCKS)
    k_wq_resident(const float* __restrict__ x, int64_t C, int64_t grows, int G, uint32_t wait_extra,
                  uint32_t spin_limit, uint32_t* __restrict__ wsu, float* __restrict__ ts, uint32_t base,
                  uint8_t* __restrict__ codes, uint8_t* __restrict__ sf, uint8_t* __restrict__ out_c,
                  uint8_t* __restrict__ out_s) {
  using namespace wr;
  __shared__ __attribute__((aligned(16))) uint8_t lq[TC * TR];       // MXFP8 [column][32 rows]
  __shared__ __attribute__((aligned(16))) uint8_t lcode[TR * TC / 2];  // NVFP4 codes [row][128 bytes]
  __shared__ __attribute__((aligned(16))) uint8_t lsf[TR * TC / 16];   // NVFP4 scale bytes [row][16]
  __shared__ uint8_t lmxs[TC];                                         // MX scale byte of each column
  __shared__ float s_red[WAVES];
  __shared__ float s_S[2];  // tensor scales of groups g (slot g & 1) and g + 1
  // per slot: 1 / (e4m3(c) S) for every scale byte c (c = 127, a NaN code,
  // as infinity), and 1 / (6 S)
  __shared__ float s_inv[2][128];
  __shared__ float s_r6[2];
  const uint32_t n_tile = gridDim.x;
  const int tid = threadIdx.x, l = tid & 63, cg = l & 7, rg = l >> 3;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t key0 = fmix32(base);
  // this workgroup's tile: 8 consecutive tiles run on 8 XCDs; each XCD takes
  // runs of 4 row-adjacent tiles (the 128 rows of four MX blocks)
  const uint32_t ti = blockIdx.x, q = ti >> 3, quad = (q >> 2) * 8 + (ti & 7);
  // (the quotient through readfirstlane: the division runs on the VALU, and
  // the tile's row and column block are uniform, kept in scalar registers)
  const uint32_t n_cb = (uint32_t)(C / TC), rq = __builtin_amdgcn_readfirstlane(quad / n_cb), cb = quad - rq * n_cb;
  const int64_t rt0 = (int64_t)(4 * rq + (q & 3)) * TR, c0 = (int64_t)cb * TC;
  const int64_t lrow = rt0 + 4 * rg, lcol = c0 + 64 * w + 8 * cg;  // the lane's first row (in its group) and column

  using Buf = f32x4[8];  // [row i][half h] at 2 i + h
  // (buffer accesses off one descriptor per group and 32-bit offsets: a
  // group's tensors stay below 2 GB, checked on the host)
  const uint32_t ld_off = (uint32_t)(lrow * C + lcol) * 4u;
  auto load = [&](int g, Buf& b) {
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(x + (int64_t)g * grows * C, (uint64_t)grows * C * 4);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(rx, ld_off, (uint32_t)(i * C * 4 + 16 * h), 0);
        b[2 * i + h] = f32x4{__uint_as_float(v[0]), __uint_as_float(v[1]), __uint_as_float(v[2]), __uint_as_float(v[3])};
      }
  };
  auto tile_max = [&](const Buf& b) {  // wave maximum to s_red[w]
    float m = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k)
      m = fmaxf(m, fmaxf(fmaxf(fabsf(b[k][0]), fabsf(b[k][1])), fmaxf(fabsf(b[k][2]), fabsf(b[k][3]))));
    m = wave_max(m);
    if (l == 0) s_red[w] = m;
  };
  // (thread 0, after a barrier) this tile's maximum of group g, marked present
  auto publish = [&](int g) {
    if (tid == 0) {
      const float mm = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
      __hip_atomic_store(wsu + (size_t)g * n_tile + ti, __float_as_uint(mm) | 0x80000000u, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    }
  };
  // (wave 0) group g's tensor scale once every tile's maximum is present;
  // after one give-up the workgroup stops waiting (a launch that cannot hold
  // all its workgroups then ends in one spin limit, not one per group)
  bool gave_up = false;
  auto take_scale = [&](int g) {
    const uint32_t* part = wsu + (size_t)g * n_tile;
    uint32_t spins = 0, mx = 0;
    bool all = false;
    while (true) {
      uint32_t v[MAX_TILES / 64];
#pragma unroll
      for (int j = 0; j < MAX_TILES / 64; ++j) {
        const uint32_t k = (uint32_t)(l + 64 * j);
        v[j] = k < n_tile ? __hip_atomic_load(part + k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0x80000000u;
      }
      bool ok = true;
      mx = 0;
#pragma unroll
      for (int j = 0; j < MAX_TILES / 64; ++j) {
        ok = ok && (v[j] >> 31) != 0u;
        mx = max(mx, v[j] & 0x7FFFFFFFu);
      }
      all = __all(ok) && wait_extra == 0u;
      if (all || gave_up || ++spins >= spin_limit) break;
      __builtin_amdgcn_s_sleep(8);
    }
    if (!all) {
      gave_up = true;
      if (l == 0) atomicOr(&g_dev_err, MOE4_DEVERR_WAIT);
    }
    const float a = __uint_as_float(wave_umax(mx));
    const float sv = a / (6.0f * 448.0f);
    const float S = (sv == 0.0f) ? 1.0f : sv;
    if (l == 0) {
      s_S[g & 1] = S;
      s_r6[g & 1] = 1.0f / (6.0f * S);
      if (ti == 0) ts[g] = S;
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int c = l + 64 * k;
      s_inv[g & 1][c] = c == 127 ? __builtin_inff() : 1.0f / (e4m3_to_f32((uint32_t)c) * S);
    }
  };
  // NVFP4 mode 6 of the lane's 4 x 8 values, then the SR MXFP8 bytes of the
  // transposed copy, both staged in LDS
  auto encode = [&](int g, const Buf& b, float S_in) {
    int lx = l;
    asm volatile("" : "+v"(lx));  // (as in store: LDS addresses made here)
    const int cg = lx & 7, rg = lx >> 3;
    const float S = __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(S_in)));  // (wave-uniform)
    const float d6 = 6.0f * S;
    const float* inv_tab = s_inv[g & 1];
    const float r6 = __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(s_r6[g & 1])));
    // a * fl(1 / d6) lies within 3 ulps of fl(a / d6) when d6 and its
    // reciprocal are normal: then if the E4M3 codes of the product 4 ulps down
    // and 4 ulps up agree, fl(a / d6) (between them) has that code too
    const bool r6_ok = d6 >= 0x1p-126f && r6 >= 0x1p-126f && r6 < __builtin_inff();
    uint32_t cw[4], scb[4];
    float am[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) am[e] = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float v[8] = {b[2 * i][0], b[2 * i][1], b[2 * i][2], b[2 * i][3],
                          b[2 * i + 1][0], b[2 * i + 1][1], b[2 * i + 1][2], b[2 * i + 1][3]};
      float a = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) a = fmaxf(a, fabsf(v[e]));
      a = fmaxf(a, lane_xor1(a));  // the block's other half
      // encode_half's steps: sc = e4m3_rne_u(a / d6) (through the product
      // check above; the division for lanes it leaves open) and the
      // reciprocal of the effective scale from the table; its zero-scale and
      // infinite-reciprocal cases (tiny values) go through encode_half
      // whenever a lane of the wave meets one
      const uint32_t ub = __float_as_uint(fminf(a * r6, 448.0f));
      const uint32_t pk = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(__uint_as_float(ub >= 4u ? ub - 4u : 0u),
                                                                   __uint_as_float(ub + 4u), 0, false);
      uint32_t sc = pk & 0xFFu;
      const bool sc_ok = r6_ok && sc == ((pk >> 8) & 0xFFu);
      if (__builtin_expect(__any(!sc_ok), 0)) {
        if (!sc_ok) sc = e4m3_rne_u(a / d6);
      }
      const float inv = inv_tab[sc];  // infinite for sc = 0 and for an underflowing e4m3(sc) S
      uint32_t q = 0u;
      if (__builtin_expect(__any(__builtin_isinf(inv)), 0)) {
        uint32_t sc2;
        q = encode_half(v, a, S, 6.0f, sc2);
      } else {
#pragma unroll
        for (int e = 0; e < 8; e += 2)
          q |= (__builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, v[e] * inv, v[e + 1] * inv, 1.0f, 0) & 0xFFu) << (4 * e);
      }
      cw[i] = q;
      scb[i] = sc;
      const int row = 4 * rg + i;
      *reinterpret_cast<uint32_t*>(lcode + row * (TC / 2) + 32 * w + 4 * cg) = q;
      if ((cg & 1) == 0) lsf[row * (TC / 16) + 4 * w + (cg >> 1)] = (uint8_t)sc;
      float q8[8];
      dequant8(q, sc, q8);
#pragma unroll
      for (int e = 0; e < 8; ++e) am[e] = fmaxf(am[e], fabsf(q8[e]));
    }
    const bool fold = fold_scale_ok(S);
    float f[8];
    int exs[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      am[e] = fmaxf(am[e], lane_xor8(am[e]));
      am[e] = max_xor32(max_xor16(am[e]));
      const int ex = mx_exponent(am[e] * S);
      const float pc = __builtin_amdgcn_ldexpf(1.0f, -ex);
      f[e] = fold ? (ex == -127 ? 0.0f : S * pc) : pc;
      exs[e] = ex;
    }
    if (rg == 0) {
#pragma unroll
      for (int e = 0; e < 8; ++e) lmxs[64 * w + 8 * cg + e] = (uint8_t)(exs[e] + 127);
    }
    uint32_t od[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) od[e] = 0u;
    const int64_t jr0 = ((int64_t)g * grows + lrow) * (C / 2) + lcol / 2;  // pair index of the lane's first pair
    // fold: fl(q * (S 2^-ex)), else fl(fl(q * S) * 2^-ex): the same values
    auto sr_rows = [&](auto val) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float q8[8];
        dequant8(cw[i], scb[i], q8);
        // (used when FAST; jr0 and C / 2 are multiples of 4: columns in steps of 8, C % 256 == 0)
        const Fmix32x4 hw((uint32_t)jr0 + (uint32_t)i * (uint32_t)(C / 2), key0);
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          uint32_t word;
          if (FAST) {
            word = hw.word(p);
          } else {
            const int64_t j = jr0 + i * (C / 2) + p;
            word = fmix32((uint32_t)j ^ fmix32(base ^ (uint32_t)((uint64_t)j >> 32)));
          }
          od[2 * p] = sr_fp8_into(od[2 * p], val(q8[2 * p], f[2 * p]), word << 16, i);
          od[2 * p + 1] = sr_fp8_into(od[2 * p + 1], val(q8[2 * p + 1], f[2 * p + 1]), word & 0xFFFF0000u, i);
        }
      }
    };
    const float Sv = fold ? 1.0f : S;  // (q * 1 is q)
    sr_rows([Sv](float q, float fe) { return (q * Sv) * fe; });
#pragma unroll
    for (int e = 0; e < 8; ++e) *reinterpret_cast<uint32_t*>(lq + (64 * w + 8 * cg + e) * TR + 4 * rg) = od[e];
  };
  using v4u = __attribute__((ext_vector_type(4))) unsigned int;
  // (waves 1-3) the staged tile of group g in runs of 64 pieces of one kind,
  // run r = (w - 1) + 3 k: 8 runs of MXFP8 codes (a column's 32 rows as two
  // 16-byte pieces), 4 of NVFP4 codes (16 bytes of a row), 4 of MX scale
  // bytes (one per column) and half a run of NVFP4 scale bytes (16 per row).
  // Each wave's runs are compile-time constants (one instantiation per
  // wave), so no run test is kept live across the rounds.  Offsets are 24-bit
  // products: a group's tile grid has at most 768 tiles of 32 x 256, so rows
  // and columns stay below 2^23.
  auto store_run = [&](auto run_c, int64_t gel, int li) {
    constexpr int run = decltype(run_c)::value;
    const int it = 64 * run + li;
    if constexpr (run < 8) {
      const int col = it >> 1, h = it & 1;
      const u32x4 v = *reinterpret_cast<const u32x4*>(lq + col * TR + 16 * h);
      __builtin_amdgcn_raw_buffer_store_b128(v4u{v[0], v[1], v[2], v[3]}, make_rsrc(out_c + gel, (uint64_t)grows * C),
                                             __umul24((uint32_t)(c0 + col), (uint32_t)grows) + (uint32_t)(rt0 + 16 * h),
                                             0, 0);
    } else if constexpr (run < 12) {
      const int jt = it - 512, row = jt >> 3, h = jt & 7;
      const u32x4 v = *reinterpret_cast<const u32x4*>(lcode + row * (TC / 2) + 16 * h);
      __builtin_amdgcn_raw_buffer_store_b128(v4u{v[0], v[1], v[2], v[3]},
                                             make_rsrc(codes + gel / 2, (uint64_t)grows * C / 2),
                                             __umul24((uint32_t)(rt0 + row), (uint32_t)(C / 2)) +
                                                 (uint32_t)(c0 / 2 + 16 * h),
                                             0, 0);
    } else if constexpr (run < 16) {
      const int col = it - 768;
      __builtin_amdgcn_raw_buffer_store_b8(lmxs[col], make_rsrc(out_s + gel / 32, (uint64_t)grows * C / 32),
                                           __umul24((uint32_t)(c0 + col), (uint32_t)(grows / 32)) +
                                               (uint32_t)(rt0 / 32),
                                           0, 0);
    } else if constexpr (run == 16) {
      if (li < TR) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(lsf + li * (TC / 16));
        __builtin_amdgcn_raw_buffer_store_b128(v4u{v[0], v[1], v[2], v[3]},
                                               make_rsrc(sf + gel / 16, (uint64_t)grows * C / 16),
                                               __umul24((uint32_t)(rt0 + li), (uint32_t)(C / 16)) +
                                                   (uint32_t)(c0 / 16),
                                               0, 0);
      }
    }
  };
  auto store = [&](int g) {
    // (the lane index passes through an empty asm so that the addresses
    // below are made here, not kept live across the rounds)
    int li = l;
    asm volatile("" : "+v"(li));
    const int64_t gel = (int64_t)g * grows * C;  // the group's first element
    using std::integral_constant;
    if (w == 1) {
      store_run(integral_constant<int, 0>{}, gel, li);
      store_run(integral_constant<int, 3>{}, gel, li);
      store_run(integral_constant<int, 6>{}, gel, li);
      store_run(integral_constant<int, 9>{}, gel, li);
      store_run(integral_constant<int, 12>{}, gel, li);
      store_run(integral_constant<int, 15>{}, gel, li);
    } else if (w == 2) {
      store_run(integral_constant<int, 1>{}, gel, li);
      store_run(integral_constant<int, 4>{}, gel, li);
      store_run(integral_constant<int, 7>{}, gel, li);
      store_run(integral_constant<int, 10>{}, gel, li);
      store_run(integral_constant<int, 13>{}, gel, li);
      store_run(integral_constant<int, 16>{}, gel, li);
    } else {
      store_run(integral_constant<int, 2>{}, gel, li);
      store_run(integral_constant<int, 5>{}, gel, li);
      store_run(integral_constant<int, 8>{}, gel, li);
      store_run(integral_constant<int, 11>{}, gel, li);
      store_run(integral_constant<int, 14>{}, gel, li);
    }
  };
  // round g: X holds group g (its tensor scale in s_S[g & 1]), Y group g + 1
  // (its maximum published), Z group g + 2 and V group g + 3 (loads may be in
  // flight).  Every wave loads at the same point, unconditionally (past the
  // last group it reloads the last one), so no register copies wait for
  // those loads; wave 0 loads after its poll, so the poll never queues behind
  // them.
  auto round = [&](int g, Buf& X, Buf& Y, Buf& Z, Buf& V) {
    const bool has1 = g + 1 < G, has2 = g + 2 < G;
    if (has2) tile_max(Z);
    __syncthreads();
    if (w == 0 && has2) publish(g + 2);
    encode(g, X, s_S[g & 1]);
    __syncthreads();
    if (w != 0) store(g);
    else if (has1) take_scale(g + 1);  // (published a round ago)
    load(g + 4 < G ? g + 4 : G - 1, X);  // X is free: group g + 4
  };
  Buf A, B, Cb, D;
  load(0, A);
  load(G > 1 ? 1 : 0, B);
  load(G > 2 ? 2 : G - 1, Cb);
  load(G > 3 ? 3 : G - 1, D);
  tile_max(A);
  __syncthreads();
  if (w == 0) publish(0);
  __syncthreads();  // s_red is free again
  if (G > 1) tile_max(B);
  __syncthreads();
  if (w == 0) {
    if (G > 1) publish(1);
    take_scale(0);
  }
  __syncthreads();  // s_red free, s_S[0] set
  for (int g = 0; g < G; g += 4) {
    round(g, A, B, Cb, D);
    if (g + 1 < G) round(g + 1, B, Cb, D, A);
    if (g + 2 < G) round(g + 2, Cb, D, A, B);
    if (g + 3 < G) round(g + 3, D, A, B, Cb);
  }
}

__global__ void k_dequant(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ sf,
                          const float* __restrict__ ts, int ts_per_group, const int32_t* __restrict__ goff,
                          int G, int64_t rows, int64_t cols, float* __restrict__ out) {
  const int64_t nbr = cols / 16;
  const int64_t blk = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (blk >= rows * nbr) return;
  const int64_t r = blk / nbr;
  const float S = ts[ts_per_group ? group_of_row(goff, G, r) : 0];
  const float scf = e4m3_to_f32(sf[blk]);
  const float mant = mant_factor(scf);
  u32x2 q = *reinterpret_cast<const u32x2*>(codes + blk * 8);
  float* o = out + blk * 16;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t byte = (q[i >> 2] >> (8 * (i & 3))) & 0xFFu;
    f32x2 p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(byte, scf, 0);
    float p0 = scf == 0.0f ? 0.0f * p[0] : p[0] * mant;
    float p1 = scf == 0.0f ? 0.0f * p[1] : p[1] * mant;
    o[2 * i] = p0 * S;
    o[2 * i + 1] = p1 * S;
  }
}

__global__ void k_silu_eval(const uint16_t* __restrict__ u, int64_t n, float* __restrict__ so,
                            float* __restrict__ dso, const float* __restrict__ tabs) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  uint32_t b = u[i];
  if (so) so[i] = act_eval<false>(b, tabs);
  if (dso) dso[i] = act_eval<true>(b, tabs + ACT_TAB);
}

}  // namespace moe4

using namespace moe4;

extern "C" size_t nvfp4_quant_46_ws_bytes(int32_t n_groups) {
  const int g = n_groups > 0 ? n_groups : 1;
  return (size_t)g * amax_slots(g) * sizeof(uint32_t);
}

extern "C" int nvfp4_quant_46(const void* x, int dtype, int64_t rows, int64_t cols,
                              const int32_t* group_row_off, int32_t n_groups, int mode, int pre_op,
                              uint8_t* codes, uint8_t* sf, float* tensor_scale,
                              void* ws, size_t ws_bytes, void* stream) {
  MOE4_REQUIRE(dtype == MOE4_BF16 || dtype == MOE4_F32, MOE4_EINVAL, "nvfp4_quant_46: dtype must be BF16 or F32");
  MOE4_REQUIRE(mode == MOE4_NVFP4_6 || mode == MOE4_NVFP4_4OVER6, MOE4_EINVAL, "nvfp4_quant_46: bad mode");
  MOE4_REQUIRE(pre_op == MOE4_PRE_NONE ||
                   ((pre_op == MOE4_PRE_SILU || pre_op == MOE4_PRE_SILU_AMAX) && dtype == MOE4_BF16),
               MOE4_EINVAL, "nvfp4_quant_46: pre_op SILU needs bf16 input");
  MOE4_REQUIRE(rows >= 0 && cols > 0 && cols % 16 == 0, MOE4_EINVAL, "nvfp4_quant_46: cols must be a positive multiple of 16");
  MOE4_REQUIRE(n_groups >= 1 && (group_row_off != nullptr || n_groups == 1), MOE4_EINVAL,
               "nvfp4_quant_46: n_groups >= 1, and group_row_off is required when n_groups > 1");
  MOE4_REQUIRE(tensor_scale && ws, MOE4_EINVAL, "nvfp4_quant_46: NULL pointer");
  MOE4_REQUIRE(rows == 0 || (x && codes && sf), MOE4_EINVAL, "nvfp4_quant_46: NULL pointer");
  MOE4_REQUIRE(aligned16(x) && aligned16(codes), MOE4_EALIGN, "nvfp4_quant_46: x and codes must be 16-byte aligned");
  MOE4_REQUIRE(ws_bytes >= nvfp4_quant_46_ws_bytes(n_groups), MOE4_EWORKSPACE, "nvfp4_quant_46: workspace too small");
  hipStream_t s = as_stream(stream);
  const float* tab = nullptr;
  const bool amax_given = pre_op == MOE4_PRE_SILU_AMAX;  // ws already holds the group amax bits
  if (amax_given) pre_op = MOE4_PRE_SILU;
  if (pre_op == MOE4_PRE_SILU) {
    int rc = act_tables(&tab);
    if (rc) return rc;
  }
  uint32_t* amax = static_cast<uint32_t*>(ws);
  const int G = n_groups;
  // (with the amax given, ws holds one word per group; the walk uses slots)
  const int slots = amax_given ? 1 : amax_slots(G);
  if (!amax_given)
    hipLaunchKernelGGL(k_zero_u32, dim3((G * slots + 255) / 256), dim3(256), 0, s, amax, G * slots);
  if (rows > 0 && !amax_given) {
    const dim3 grid = walk_grid(rows * cols);
    if (dtype == MOE4_BF16 && pre_op == MOE4_PRE_SILU)
      hipLaunchKernelGGL((k_amax<MOE4_BF16, true>), grid, dim3(QTHREADS), 0, s, x, rows, cols, group_row_off, G, amax, tab,
                         slots);
    else if (dtype == MOE4_BF16)
      hipLaunchKernelGGL((k_amax<MOE4_BF16, false>), grid, dim3(QTHREADS), 0, s, x, rows, cols, group_row_off, G, amax, tab,
                         slots);
    else
      hipLaunchKernelGGL((k_amax<MOE4_F32, false>), grid, dim3(QTHREADS), 0, s, x, rows, cols, group_row_off, G, amax, tab,
                         slots);
  }
  const float m448 = (mode == MOE4_NVFP4_4OVER6) ? 4.0f * 448.0f : 6.0f * 448.0f;
  hipLaunchKernelGGL(k_tensor_scale, dim3((G + 255) / 256), dim3(256), 0, s, amax, G, m448, tensor_scale, slots);
  if (rows > 0) {
    const int64_t nblk = rows * (cols / 16);
    dim3 grid((unsigned)((nblk + ENC_THREADS - 1) / ENC_THREADS));
    const bool four6 = mode == MOE4_NVFP4_4OVER6;
    if (dtype == MOE4_BF16 && pre_op == MOE4_PRE_SILU)
      launch_encode<MOE4_BF16, true>(four6, grid, s, x, rows, cols, group_row_off, G, tensor_scale, codes, sf, tab);
    else if (dtype == MOE4_BF16)
      launch_encode<MOE4_BF16, false>(four6, grid, s, x, rows, cols, group_row_off, G, tensor_scale, codes, sf, tab);
    else
      launch_encode<MOE4_F32, false>(four6, grid, s, x, rows, cols, group_row_off, G, tensor_scale, codes, sf, tab);
  }
  return check_launch("nvfp4_quant_46");
}

// ------------------------------------------------ allocation-free variant
// nvfp4_quant_46's scratch (the per-group amax words) in a static device
// array, for callers that cannot allocate.  In host code `scratch` names a
// host-side stand-in: kernels get the device address that
// hipGetSymbolAddress gives, looked up once per device (that device current)
// and kept in g_scratch_ptr.
constexpr int NOALLOC_MAX_GROUPS = 4096;
static __device__ __align__(256) uint32_t scratch[NOALLOC_MAX_GROUPS];
static std::mutex g_scratch_mu;
static uint32_t* g_scratch_ptr[64];

static int scratch_device_ptr(uint32_t** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return fail(MOE4_EHIP, "hipGetDevice failed");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(MOE4_EHIP, std::string("hipGetSymbolAddress(scratch) failed: ") + hipGetErrorString(e));
    g_scratch_ptr[dev] = static_cast<uint32_t*>(p);
  }
  *out = g_scratch_ptr[dev];
  return MOE4_OK;
}

extern "C" int nvfp4_quant_46_noalloc(const void* x, int dtype, int64_t rows, int64_t cols,
                                      const int32_t* group_row_off, int32_t n_groups, int mode, int pre_op,
                                      uint8_t* codes, uint8_t* sf, float* tensor_scale, void* stream) {
  MOE4_REQUIRE(pre_op == MOE4_PRE_NONE || pre_op == MOE4_PRE_SILU, MOE4_EINVAL,
               "nvfp4_quant_46_noalloc: pre_op must be MOE4_PRE_NONE or MOE4_PRE_SILU");
  MOE4_REQUIRE(n_groups >= 1 && n_groups <= NOALLOC_MAX_GROUPS, MOE4_EINVAL,
               "nvfp4_quant_46_noalloc: n_groups must be in [1, 4096] (the static scratch holds 4096 groups)");
  uint32_t* ws = nullptr;
  int rc = scratch_device_ptr(&ws);
  if (rc) return rc;
  // nvfp4_quant_46 clears its amax words (at most 4096) with a kernel before use
  return nvfp4_quant_46(x, dtype, rows, cols, group_row_off, n_groups, mode, pre_op, codes, sf, tensor_scale, ws,
                        nvfp4_quant_46_ws_bytes(n_groups), stream);
}

// Workgroups of k_wq_resident the device holds at once (its launch needs
// them all resident), per device and instantiation.
static int64_t wq_resident_capacity(bool fast) {
  static int64_t cap[64][2];
  static std::mutex mu;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  std::lock_guard<std::mutex> lock(mu);
  if (cap[dev][fast] == 0) {
    int nb = 0;
    const hipError_t e = fast ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, k_wq_resident<true>, wr::THREADS, 0)
                              : hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, k_wq_resident<false>, wr::THREADS, 0);
    cap[dev][fast] = (e == hipSuccess && nb > 0) ? (int64_t)nb * cu_count_q() : -1;
  }
  return cap[dev][fast];
}

// Workspace (32-bit words, cleared before the launch): k_wq_resident keeps
// its tiles' maxima there (n_tile <= MAX_TILES words per group);
// k_encode_requant_T uses the first 2 G + 1 words (amax bits [G], finished
// amax tiles [G], the ticket counter).
extern "C" size_t nvfp4_quant_requant_T_ws_bytes(int32_t n_groups) {
  const size_t g = (size_t)(n_groups > 0 ? n_groups : 1);
  return g * wr::MAX_TILES * sizeof(uint32_t);  // (>= the ticketed kernel's 2 g + 1 words)
}

extern "C" int nvfp4_quant_requant_T(const float* x, int64_t rows, int64_t cols, int32_t n_groups, uint8_t* codes,
                                     uint8_t* sf, float* tensor_scale, uint64_t seed, uint32_t stream_id,
                                     uint8_t* mx_codes, uint8_t* mx_sf, void* ws, size_t ws_bytes, void* stream) {
  MOE4_REQUIRE(rows >= 0 && cols > 0 && cols % 32 == 0, MOE4_EINVAL,
               "nvfp4_quant_requant_T: cols must be a positive multiple of 32");
  MOE4_REQUIRE(n_groups >= 1 && rows % n_groups == 0 && (rows / n_groups) % 32 == 0, MOE4_EINVAL,
               "nvfp4_quant_requant_T: rows must split into n_groups equal groups of a multiple of 32 rows");
  MOE4_REQUIRE(rows / n_groups < ((int64_t)1 << 31) / 2 && rows < ((int64_t)1 << 31), MOE4_EINVAL,
               "nvfp4_quant_requant_T: too many rows");
  MOE4_REQUIRE(tensor_scale && ws, MOE4_EINVAL, "nvfp4_quant_requant_T: NULL pointer");
  MOE4_REQUIRE(rows == 0 || (x && codes && sf && mx_codes && mx_sf), MOE4_EINVAL, "nvfp4_quant_requant_T: NULL pointer");
  MOE4_REQUIRE(aligned16(x) && aligned16(codes) && aligned16(mx_codes), MOE4_EALIGN,
               "nvfp4_quant_requant_T: x, codes and mx_codes must be 16-byte aligned");
  MOE4_REQUIRE(ws_bytes >= nvfp4_quant_requant_T_ws_bytes(n_groups), MOE4_EWORKSPACE,
               "nvfp4_quant_requant_T: workspace too small");
  hipStream_t s = as_stream(stream);
  const int G = n_groups;
  const int64_t grows = rows / G;
  uint32_t* wsu = static_cast<uint32_t*>(ws);
  const int n_words = 2 * G + 1;
  hipLaunchKernelGGL(k_zero_u32, dim3((n_words + 255) / 256), dim3(256), 0, s, wsu, n_words);
  if (rows == 0) {  // empty groups: tensor scale 1
    hipLaunchKernelGGL(k_tensor_scale, dim3((G + 255) / 256), dim3(256), 0, s, wsu, G, 6.0f * 448.0f, tensor_scale);
    return check_launch("nvfp4_quant_requant_T");
  }
  const bool forced = force_wait_timeout();
  const uint32_t base = sr_base_key(seed, stream_id);
  // one HBM read when every tile of a group fits the chip at once
  if (grows % (4 * wr::TR) == 0 && cols % wr::TC == 0 && aligned16(sf)) {
    const int64_t n_tile = (grows / wr::TR) * (cols / wr::TC);
    const bool fast = rows * (cols / 2) <= ((int64_t)1 << 32);
    if (n_tile % 32 == 0 && n_tile <= wr::MAX_TILES && n_tile <= wq_resident_capacity(fast)) {
      auto k = fast ? k_wq_resident<true> : k_wq_resident<false>;
      const int64_t n_zero = (int64_t)G * n_tile;
      hipLaunchKernelGGL(k_zero_u32, dim3((unsigned)((n_zero + 255) / 256)), dim3(256), 0, s, wsu, (int)n_zero);
      hipLaunchKernelGGL(k, dim3((unsigned)n_tile), dim3(wr::THREADS), 0, s, x, cols, grows, G, forced ? 1u : 0u,
                         forced ? wq::FORCED_SPIN_LIMIT : wq::SPIN_LIMIT, wsu, tensor_scale, base, codes, sf, mx_codes,
                         mx_sf);
      return check_launch("nvfp4_quant_requant_T");
    }
  }
  const int64_t n_ct = (cols + rq::COLS - 1) / rq::COLS, n_item = (grows + rq::ROWS - 1) / rq::ROWS * n_ct;
  const int64_t n_total = (int64_t)G * n_item;
  const int64_t slots = (int64_t)cu_count_q() * 2;  // two 64 KB-LDS workgroups per CU
  MOE4_REQUIRE(2 * n_total + slots < ((int64_t)1 << 31), MOE4_EINVAL, "nvfp4_quant_requant_T: tensor too large");
  const int64_t grid = 2 * n_total < slots ? 2 * n_total : slots;
  hipLaunchKernelGGL(k_encode_requant_T, dim3((unsigned)grid), dim3(rq::THREADS), 0, s, x, cols, grows, G,
                     (uint32_t)n_ct, (uint32_t)n_item, forced ? 1u : 0u,
                     forced ? wq::FORCED_SPIN_LIMIT : wq::SPIN_LIMIT, wsu, tensor_scale, base, codes, sf, mx_codes,
                     mx_sf);
  return check_launch("nvfp4_quant_requant_T");
}

extern "C" int nvfp4_dequant(const uint8_t* codes, const uint8_t* sf, const float* ts, int ts_per_group,
                             const int32_t* group_row_off, int32_t n_groups, int64_t rows, int64_t cols,
                             float* out, void* stream) {
  MOE4_REQUIRE(rows >= 0 && cols > 0 && cols % 16 == 0, MOE4_EINVAL, "nvfp4_dequant: cols must be a positive multiple of 16");
  MOE4_REQUIRE(codes && sf && ts && out, MOE4_EINVAL, "nvfp4_dequant: NULL pointer");
  MOE4_REQUIRE(!ts_per_group || (group_row_off && n_groups >= 1), MOE4_EINVAL, "nvfp4_dequant: groups needed");
  MOE4_REQUIRE(aligned16(codes) && aligned16(out), MOE4_EALIGN, "nvfp4_dequant: misaligned pointer");
  if (rows == 0) return MOE4_OK;
  const int64_t nblk = rows * (cols / 16);
  hipLaunchKernelGGL(k_dequant, dim3((unsigned)((nblk + 255) / 256)), dim3(256), 0, as_stream(stream), codes, sf,
                     ts, ts_per_group, group_row_off, n_groups, rows, cols, out);
  return check_launch("nvfp4_dequant");
}

extern "C" int moe_silu_eval(const uint16_t* u, int64_t n, float* silu_out, float* dsilu_out, void* stream) {
  MOE4_REQUIRE(n >= 0 && (n == 0 || u), MOE4_EINVAL, "moe_silu_eval: bad arguments");
  hipStream_t s = as_stream(stream);
  const float* tab = nullptr;
  int rc = act_tables(&tab);
  if (rc) return rc;
  if (n == 0) return MOE4_OK;
  hipLaunchKernelGGL(k_silu_eval, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, u, n, silu_out, dsilu_out,
                     tab);
  return check_launch("moe_silu_eval");
}
