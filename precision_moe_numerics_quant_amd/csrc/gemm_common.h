// Shared pieces of the expert-grouped GEMM kernels (gfx950).
#pragma once
#include "moe4_internal.h"

namespace moe4 {

// XCD-aware tile order.  MI355X dispatches consecutive workgroups round-robin
// over its 8 XCDs (each with its own L2); mapping workgroup b to tile
// (b % 8) * ceil(n/8) + b / 8 gives each XCD a contiguous run of tiles, so the
// tiles that share an operand slab (e.g. all N-tiles of one M-tile) run on the
// same XCD and hit the same L2.  The grid is rounded up to a multiple of 8;
// workgroups whose tile is >= n exit.
constexpr int N_XCD = 8;
__host__ __device__ inline int64_t xcd_grid(int64_t n) { return (n + N_XCD - 1) / N_XCD * N_XCD; }
__device__ inline int64_t xcd_tile(int64_t b, int64_t n) {
  const int64_t per = (n + N_XCD - 1) / N_XCD;
  return (b % N_XCD) * per + b / N_XCD;
}

// Find which expert a flat M-tile index belongs to, for rows grouped by
// off[0..E] and BM rows per tile: tiles of expert e are
// [sum_{e'<e} ceil(M_e'/BM), ...).  Executed by every wave of the block (each
// gets the same answer).  Returns false when the index is past the last tile.
__device__ inline bool find_m_tile(const int32_t* __restrict__ off, int E, int BM, int64_t tile, int& e_out,
                                   int64_t& tile_in_e) {
  const int lane = threadIdx.x & 63;
  int64_t run = 0;
  for (int e0 = 0; e0 < E; e0 += 64) {
    const int e = e0 + lane;
    int cnt = 0;
    if (e < E) {
      const int m = off[e + 1] - off[e];
      cnt = m > 0 ? (m + BM - 1) / BM : 0;
    }
    int inc = cnt;  // inclusive prefix within the wave
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      int y = __shfl_up(inc, o, 64);
      if (lane >= o) inc += y;
    }
    const int total = __shfl(inc, 63, 64);
    if (tile < run + total) {
      const bool hit = (tile < run + inc) && (tile >= run + inc - cnt);
      const unsigned long long b = __ballot(hit);
      const int src = __ffsll((long long)b) - 1;
      const int excl = __shfl(inc - cnt, src, 64);
      // wave-uniform results: keep them in scalar registers
      e_out = __builtin_amdgcn_readfirstlane(e0 + src);
      tile_in_e = __builtin_amdgcn_readfirstlane((int)(tile - run - excl));
      return true;
    }
    run += total;
  }
  return false;
}

// Buffer descriptor of a wave-uniform range (kept in scalar registers).
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint64_t bytes) {
  const uint32_t n = bytes > 0x7FFFFFF0ull ? 0x7FFFFFF0u : (uint32_t)bytes;
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  // readfirstlane yields a signed 32-bit int: go through uint32_t so that the
  // low word is zero-extended (a sign-extended low word would corrupt the base)
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  const uint64_t au = ((uint64_t)hi << 32) | (uint64_t)lo;
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(au), (short)0,
                                           __builtin_amdgcn_readfirstlane((int)n), 0x00020000);
}

// Element i of a launch-constant int32 array, through the constant address
// space: a uniform index then always gives a scalar load (a vector load would
// make the wave wait for all its outstanding loads and stores).
__device__ inline int32_t ld_const(const int32_t* p, int i) {
  return reinterpret_cast<const __attribute__((address_space(4))) int32_t*>(
      reinterpret_cast<uintptr_t>(p))[i];
}

// Cursor over the m-tiles of the experts in order: (expert, its first m-tile).
template <int TM>
struct MtCursor {
  int e = 0;
  uint32_t first = 0;  // flat index of expert e's first m-tile
  // advance to the expert holding flat m-tile mi; false past the last one.
  // The offsets come through scalar loads: a vector load here would make the
  // wave wait for all its outstanding loads (or stores) first.
  __device__ bool seek(const int32_t* __restrict__ off, int E, uint32_t mi) {
    while (e < E) {
      const int32_t o0 = ld_const(off, e), o1 = ld_const(off, e + 1);
      const uint32_t n = (uint32_t)((o1 - o0 + TM - 1) / TM);
      if (mi < first + n) return true;
      first += n;
      ++e;
    }
    return false;
  }
};

// Tile order of the persistent warp-specialised GEMMs over (m-tile, n-tile)
// (forward and dgrad).  The 8 XCDs work side by side on one
// band of SM = (8 / xb) pm m-tiles at a time: XCD x takes the pm x pn
// rectangle (x / xb, x % xb) of the band (pn n-tiles, n fastest), its
// workgroups the rectangle's tiles in turn, then the next band.  Each XCD's
// L2 then holds pm A row blocks and pn B row blocks per band, and the XCDs
// read the same experts' B rows at about the same time (shared in the
// Infinity Cache).  q: the XCD's own tile counter.
struct DgSplit {
  uint32_t pm, pn, xb;
  __device__ bool tile(uint32_t x, uint32_t q, uint32_t n_mt, uint32_t n_nt, uint32_t& mi, uint32_t& nt) const {
    const uint32_t ppn = pm * pn, sb = q / ppn, r = q - sb * ppn, a = r / pn;
    mi = sb * (8 / xb) * pm + (x / xb) * pm + a;
    nt = (x % xb) * pn + (r - a * pn);
    return mi < n_mt && nt < n_nt;
  }
};

// The rectangle with the fewest operand rows per tile (TM-row A blocks,
// TN-row B blocks), counting n-tiles past n_nt as waste: pm = 32 / pn (one
// tile per workgroup of an XCD of 32 CUs at a time; 1 for pn >= 32).  A B row (the
// requantised weights, met first in HBM) counts three A rows: measured on the
// layer's dgrads, the order with the fewest B rows per XCD is the
// fastest of those with the same total.
inline DgSplit dg_split(int64_t n_nt, int tm, int tn) {
  DgSplit best{1, 1, 1};
  double best_cost = 1e300;
  for (uint32_t xb = 1; xb <= 8; xb *= 2) {
    const uint32_t pn = (uint32_t)((n_nt + xb - 1) / xb);
    const uint32_t pm = pn >= 32 ? 1 : 32 / pn;
    const double cost =
        ((double)pm * tm + 3.0 * pn * tn) / ((double)pm * pn) * ((double)xb * pn / (double)n_nt);
    if (cost < best_cost) {
      best_cost = cost;
      best = DgSplit{pm, pn, xb};
    }
  }
  return best;
}

}  // namespace moe4
