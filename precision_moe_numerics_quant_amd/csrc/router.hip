// The BF16 router in front of the expert layer (gfx950): its GEMM and its
// backward.  The pages route each token to 8 of 384 experts (fourweekmba.com
// page, "Update") and keep some activations in BF16 (lhc.media page,
// paragraph on the precisions that remain); the router itself is read as a
// linear map in BF16, logits = x . W_r^T, float32 out.
//
//   k_router_gemm      logits [T, E] = x [T, d] . W_r [E, d]^T: bf16 MFMA
//                      (v_mfma_f32_32x32x16_bf16), float32 accumulation, 128 x
//                      128 tiles (T x E), K slabs of 64 through two LDS buffers.
//   k_unpermute_router the un-permuting sum of the expert path's input
//                      gradient plus the router's: dx[t] = bf16(sum_j dXp[row]
//                      + sum_j dz[t, e_j] * W_r[e_j]), in that float32 order.
//   router wgrad       dW_r [E, d] = sum over the tokens routed to e of
//                      dz[t, e] * x[t]: sparse (k of E logits per token carry a
//                      gradient), so a gather-reduce over each expert's routed
//                      rows, not a dense GEMM.  Each expert's rows are cut into
//                      chunks of 128, so a popular expert (routing is skewed:
//                      one expert can hold most tokens) spreads over the whole
//                      chip: k_router_wgrad_chunks numbers the chunks,
//                      k_router_wgrad_part sums each (chunk, 512 columns) into
//                      a float32 partial row, k_router_wgrad_sum adds each
//                      expert's partials in chunk order (deterministic).
#include "gemm_common.h"
#include "moe4_internal.h"

namespace moe4 {

// This file's device-side error word (moe4_debug_check reads and clears it).
static __device__ uint32_t g_dev_err;
uint32_t take_dev_err_router() { return take_device_word(&g_dev_err); }

namespace rg {
constexpr int TM = 128, TN = 128, BK = 64, NT = 256;
constexpr int ROW_B = BK * 2;               // bytes per LDS row (64 bf16)
constexpr int TILE_B = TM * ROW_B;          // one operand's slab (16 KB)
// 16-byte chunk c of row r sits at chunk c ^ (r & 7): 8 consecutive rows
// reading the same logical chunk hit 8 different bank groups
__device__ inline int swz(int r, int c) { return c ^ (r & 7); }
}  // namespace rg

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__global__ void __launch_bounds__(rg::NT, 2)
    k_router_gemm(const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, int64_t T, int E, int64_t d,
                  float* __restrict__ out) {
  using namespace rg;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][2][TILE_B];   // [buffer][operand][slab]
  const int tid = threadIdx.x, l = tid & 63, wv = tid >> 6;
  const int64_t n_et = (E + TN - 1) / TN;
  const int64_t tile = blockIdx.x;
  const int64_t t0 = (tile / n_et) * TM, e0 = (tile % n_et) * TN;
  // loads: thread tid takes 16-byte chunk (tid & 7) of rows tid / 8 + 32 j
  const int ch = tid & 7, rr = tid >> 3;
  u32x4 ra[4], rb[4];
  auto load = [&](int64_t k0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = rr + 32 * j;
      const int64_t ta = t0 + r, eb = e0 + r;
      ra[j] = ta < T ? *reinterpret_cast<const u32x4*>(x + ta * d + k0 + 8 * ch) : u32x4{0u, 0u, 0u, 0u};
      rb[j] = eb < E ? *reinterpret_cast<const u32x4*>(w + eb * d + k0 + 8 * ch) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = rr + 32 * j;
      *reinterpret_cast<u32x4*>(&lds[buf][0][r * ROW_B + 16 * swz(r, ch)]) = ra[j];
      *reinterpret_cast<u32x4*>(&lds[buf][1][r * ROW_B + 16 * swz(r, ch)]) = rb[j];
    }
  };
  // wave (wm, wn) owns the 64 x 64 block; 2 x 2 MFMA tiles of 32 x 32
  const int wm = (wv >> 1) * 64, wn = (wv & 1) * 64;
  const int li = l & 31, g = l >> 5;
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};
  const int nk = (int)(d / BK);
  load(0);
  store(0);
  __syncthreads();
  for (int s = 0; s < nk; ++s) {
    const int buf = s & 1;
    if (s + 1 < nk) load((int64_t)(s + 1) * BK);       // in flight during this slab's MFMAs
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      // lane (li, g) holds 8 consecutive k of row li: k = 16 kk + 8 g .. + 7
      const int c = 2 * kk + g;
      bf16x8 a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r = wm + 32 * i + li;
        a[i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(&lds[buf][0][r * ROW_B + 16 * swz(r, c)]));
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int r = wn + 32 * j + li;
        b[j] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(&lds[buf][1][r * ROW_B + 16 * swz(r, c)]));
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    if (s + 1 < nk) store(buf ^ 1);                     // the other buffer: last read two slabs ago
    __syncthreads();
  }
  // C[t0 + wm + 32 i + row][e0 + wn + 32 j + li], row = (v / 4) * 8 + 4 g + v % 4
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t col = e0 + wn + 32 * j + li;
      if (col >= E) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t row = t0 + wm + 32 * i + (v >> 2) * 8 + 4 * g + (v & 3);
        if (row < T) out[row * E + col] = acc[i][j][v];
      }
    }
}

// idx clamped to [0, n); a clamp is reported
__device__ inline int64_t clamp_rt(int64_t i, int64_t n) {
  if (i < 0 || i >= n) {
    atomicOr(&g_dev_err, MOE4_DEVERR_INDEX);
    return i < 0 ? 0 : n - 1;
  }
  return i;
}

constexpr int RMAXK = 16;

// One thread per (token, 4 columns).
__global__ void __launch_bounds__(256) k_unpermute_router(const float* __restrict__ dxp, const int32_t* __restrict__ inv,
                                                          int64_t T, int k, int64_t d, int64_t n_rows,
                                                          const float* __restrict__ dlogits,
                                                          const int32_t* __restrict__ idx, int E,
                                                          const uint16_t* __restrict__ w, uint16_t* __restrict__ dx) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t nq = d / 4;
  if (q >= T * nq) return;
  const int64_t t = q / nq, c = (q % nq) * 4;
  f32x4 v[RMAXK];
  u32x2 wv[RMAXK];
  float dz[RMAXK];
#pragma unroll
  for (int j = 0; j < RMAXK; ++j) {
    if (j < k) {
      const int64_t row = clamp_rt(inv[t * k + j], n_rows);
      const int64_t e = clamp_rt(idx[t * k + j], E);
      v[j] = *reinterpret_cast<const f32x4*>(dxp + row * d + c);
      wv[j] = *reinterpret_cast<const u32x2*>(w + e * d + c);
      dz[j] = dlogits[t * E + e];
    }
  }
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int j = 0; j < RMAXK; ++j)
    if (j < k) {
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = acc[i] + v[j][i];
    }
#pragma unroll
  for (int j = 0; j < RMAXK; ++j)
    if (j < k) {
      const float w0 = bf16_bits_to_f32(wv[j][0] & 0xFFFFu), w1 = bf16_bits_to_f32(wv[j][0] >> 16);
      const float w2 = bf16_bits_to_f32(wv[j][1] & 0xFFFFu), w3 = bf16_bits_to_f32(wv[j][1] >> 16);
      acc[0] = acc[0] + dz[j] * w0;
      acc[1] = acc[1] + dz[j] * w1;
      acc[2] = acc[2] + dz[j] * w2;
      acc[3] = acc[3] + dz[j] * w3;
    }
  *reinterpret_cast<u32x2*>(dx + t * d + c) = u32x2{f32_to_bf16_bits(acc[0]) | (f32_to_bf16_bits(acc[1]) << 16),
                                                    f32_to_bf16_bits(acc[2]) | (f32_to_bf16_bits(acc[3]) << 16)};
}

namespace rw {
constexpr int CH = 128;               // rows per chunk
constexpr int NW = 4, NT = 64 * NW;   // k_router_wgrad_part: 4 waves
constexpr int COLS = 512;             // ... 8 columns per lane (one 16-byte load per row)
constexpr int BATCH = 16;             // ... rows in flight per wave
constexpr int SCAN_T = 1024;          // k_router_wgrad_chunks: one workgroup
constexpr int SUM_T = 256, SUM_COLS = 4 * SUM_T;  // k_router_wgrad_sum: 4 columns per thread
}

// Chunks of the rows [off[e], off[e+1]) (a span outside [0, A] counts as clipped to it).
__device__ inline int64_t rw_chunks(const int32_t* off, int e, int64_t A) {
  int64_t n = (int64_t)off[e + 1] - off[e];
  n = n < 0 ? 0 : (n > A ? A : n);
  return (n + rw::CH - 1) / rw::CH;
}

// One workgroup: coff[e] = first chunk of expert e (exclusive prefix sum of
// the chunk counts), coff[E] = the number of chunks, chunk_e[c] = the expert
// of chunk c.  Counts past `bound` (only for offsets that are not monotone
// within [0, A]) are cut there and reported.
__global__ void __launch_bounds__(rw::SCAN_T) k_router_wgrad_chunks(const int32_t* __restrict__ off, int E, int64_t A,
                                                                    int64_t bound, int32_t* __restrict__ coff,
                                                                    int32_t* __restrict__ chunk_e) {
  using namespace rw;
  __shared__ int64_t sc[SCAN_T];
  const int tid = threadIdx.x;
  const int per = (E + SCAN_T - 1) / SCAN_T;
  const int e0 = tid * per;
  int64_t mine = 0;
  for (int i = 0; i < per; ++i)
    if (e0 + i < E) mine += rw_chunks(off, e0 + i, A);
  sc[tid] = mine;
  __syncthreads();
  for (int s = 1; s < SCAN_T; s <<= 1) {  // inclusive scan (Hillis-Steele)
    const int64_t v = tid >= s ? sc[tid - s] : 0;
    __syncthreads();
    sc[tid] += v;
    __syncthreads();
  }
  int64_t c = sc[tid] - mine;  // exclusive
  bool cut = false;
  for (int i = 0; i < per; ++i) {
    const int e = e0 + i;
    if (e >= E) break;
    coff[e] = (int32_t)(c < bound ? c : bound);
    const int64_t n = rw_chunks(off, e, A);
    for (int64_t j = 0; j < n; ++j) {
      if (c + j < bound) chunk_e[c + j] = e;
      else cut = true;
    }
    c += n;
  }
  if (tid == SCAN_T - 1) {
    coff[E] = (int32_t)(sc[tid] < bound ? sc[tid] : bound);
    cut = cut || sc[tid] > bound;
  }
  if (cut) atomicOr(&g_dev_err, MOE4_DEVERR_INDEX);
}

// Block (chunk c, column block): part[c, cb .. cb + 511] = the sum over the
// chunk's rows of dz[t, e] * x[t, cols].  Wave w takes rows w, w + 4, ... of
// the chunk (16 in flight) in row order; the four wave sums are added in wave
// order.  Rows, tokens and dz are uniform per wave (scalar loads).
__global__ void __launch_bounds__(rw::NT) k_router_wgrad_part(const uint16_t* __restrict__ x,
                                                              const float* __restrict__ dlogits,
                                                              const int32_t* __restrict__ perm,
                                                              const int32_t* __restrict__ off,
                                                              const int32_t* __restrict__ coff,
                                                              const int32_t* __restrict__ chunk_e, int64_t T, int E,
                                                              int k, int64_t d, float* __restrict__ part) {
  using namespace rw;
  __shared__ f32x4 red[NW - 1][64][2];
  const int64_t c = blockIdx.x;
  if (c >= coff[E]) return;
  const int e = chunk_e[c];
  const int64_t A = T * k;
  const int64_t r0 = (int64_t)off[e] + (c - coff[e]) * CH;
  const int64_t r_end = (int64_t)off[e + 1] < r0 + CH ? (int64_t)off[e + 1] : r0 + CH;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), l = threadIdx.x & 63;
  const int64_t col = (int64_t)blockIdx.y * COLS + 8 * l;
  const bool cok = col < d;
  f32x4 a0 = {0.0f, 0.0f, 0.0f, 0.0f}, a1 = a0;
  for (int64_t rb = r0 + w; rb < r_end; rb += NW * BATCH) {
    float dz[BATCH];
    u32x4 xv[BATCH];
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      const int64_t rr = rb + (int64_t)u * NW;
      dz[u] = 0.0f;
      xv[u] = u32x4{0u, 0u, 0u, 0u};
      if (rr < r_end) {
        const int64_t t = clamp_rt(perm[clamp_rt(rr, A)], A) / k;
        dz[u] = dlogits[t * E + e];
        if (cok) xv[u] = *reinterpret_cast<const u32x4*>(x + t * d + col);
      }
    }
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      if (rb + (int64_t)u * NW < r_end) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          a0[2 * i] = a0[2 * i] + dz[u] * bf16_bits_to_f32(xv[u][i] & 0xFFFFu);
          a0[2 * i + 1] = a0[2 * i + 1] + dz[u] * bf16_bits_to_f32(xv[u][i] >> 16);
          a1[2 * i] = a1[2 * i] + dz[u] * bf16_bits_to_f32(xv[u][2 + i] & 0xFFFFu);
          a1[2 * i + 1] = a1[2 * i + 1] + dz[u] * bf16_bits_to_f32(xv[u][2 + i] >> 16);
        }
      }
    }
  }
  if (w > 0) {
    red[w - 1][l][0] = a0;
    red[w - 1][l][1] = a1;
  }
  __syncthreads();
  if (w == 0 && cok) {
#pragma unroll
    for (int q = 0; q < NW - 1; ++q) {
      a0 = a0 + red[q][l][0];
      a1 = a1 + red[q][l][1];
    }
    f32x4* o = reinterpret_cast<f32x4*>(part + c * d + col);
    o[0] = a0;
    o[1] = a1;
  }
}

// dw[e, cols] = the sum of expert e's partial rows in chunk order (zeros for
// an expert without rows).
__global__ void __launch_bounds__(rw::SUM_T) k_router_wgrad_sum(const int32_t* __restrict__ coff,
                                                                const float* __restrict__ part, int64_t d,
                                                                float* __restrict__ dw) {
  using namespace rw;
  const int e = blockIdx.x;
  const int64_t col = (int64_t)blockIdx.y * SUM_COLS + 4 * threadIdx.x;
  if (col >= d) return;
  const int64_t c0 = coff[e], c1 = coff[e + 1];
  f32x4 s = {0.0f, 0.0f, 0.0f, 0.0f};
  int64_t c = c0;
  for (; c + 8 <= c1; c += 8) {  // eight loads in flight, added in order
    f32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = *reinterpret_cast<const f32x4*>(part + (c + u) * d + col);
#pragma unroll
    for (int u = 0; u < 8; ++u) s = s + v[u];
  }
  for (; c < c1; ++c) s = s + *reinterpret_cast<const f32x4*>(part + c * d + col);
  *reinterpret_cast<f32x4*>(dw + (int64_t)e * d + col) = s;
}

// Workspace of the router wgrad: coff [E + 1], chunk_e [bound], part [bound, d].
struct RwLayout {
  int64_t bound, off_chunk_e, off_part, bytes;
};
inline RwLayout rw_layout(int64_t T, int E, int k, int64_t d) {
  RwLayout L;
  L.bound = (T * k + rw::CH - 1) / rw::CH + E;
  L.off_chunk_e = ((int64_t)(E + 1) * 4 + 255) / 256 * 256;
  L.off_part = L.off_chunk_e + (L.bound * 4 + 255) / 256 * 256;
  L.bytes = L.off_part + L.bound * d * 4;
  return L;
}

}  // namespace moe4

using namespace moe4;

extern "C" int moe_router_logits(const uint16_t* x, const uint16_t* w, int64_t T, int32_t E, int64_t d, float* logits,
                                 void* stream) {
  MOE4_REQUIRE(T >= 0 && E >= 1 && d > 0 && d % rg::BK == 0, MOE4_EINVAL,
               "moe_router_logits: need T >= 0, E >= 1 and d a positive multiple of 64");
  MOE4_REQUIRE(w && (T == 0 || (x && logits)), MOE4_EINVAL, "moe_router_logits: NULL pointer");
  MOE4_REQUIRE(aligned16(x) && aligned16(w), MOE4_EALIGN, "moe_router_logits: x and w must be 16-byte aligned");
  if (T == 0) return MOE4_OK;
  const int64_t tiles = ((T + rg::TM - 1) / rg::TM) * ((E + rg::TN - 1) / rg::TN);
  MOE4_REQUIRE(tiles < ((int64_t)1 << 31), MOE4_EINVAL, "moe_router_logits: too large");
  hipLaunchKernelGGL(k_router_gemm, dim3((unsigned)tiles), dim3(rg::NT), 0, as_stream(stream), x, w, T, E, d, logits);
  return check_launch("moe_router_logits");
}

extern "C" int moe_unpermute_sum_router(const float* dxp, const int32_t* inv_perm, int64_t T, int32_t k, int64_t d,
                                        const float* dlogits, const int32_t* topk_idx, int32_t E, const uint16_t* w,
                                        uint16_t* dx, void* stream) {
  MOE4_REQUIRE(T >= 0 && k >= 1 && k <= RMAXK && k <= E && d > 0 && d % 4 == 0, MOE4_EINVAL,
               "moe_unpermute_sum_router: need 1 <= k <= min(E, 16) and d % 4 == 0");
  MOE4_REQUIRE(T == 0 || (dxp && inv_perm && dlogits && topk_idx && w && dx), MOE4_EINVAL,
               "moe_unpermute_sum_router: NULL pointer");
  MOE4_REQUIRE(aligned16(dxp) && ((uintptr_t)w & 7u) == 0 && ((uintptr_t)dx & 7u) == 0, MOE4_EALIGN,
               "moe_unpermute_sum_router: dxp 16-byte, w and dx 8-byte aligned");
  if (T == 0) return MOE4_OK;
  const int64_t n = T * (d / 4);
  hipLaunchKernelGGL(k_unpermute_router, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, as_stream(stream), dxp,
                     inv_perm, T, k, d, T * k, dlogits, topk_idx, E, w, dx);
  return check_launch("moe_unpermute_sum_router");
}

extern "C" size_t moe_router_wgrad_ws_bytes(int64_t T, int32_t E, int32_t k, int64_t d) {
  if (T < 0 || E < 1 || k < 1 || d < 1) return 0;
  return (size_t)rw_layout(T, E, k, d).bytes;
}

extern "C" int moe_router_wgrad(const uint16_t* x, const float* dlogits, const int32_t* perm, const int32_t* expert_off,
                                int64_t T, int32_t E, int32_t k, int64_t d, float* dw, void* ws, size_t ws_bytes,
                                void* stream) {
  MOE4_REQUIRE(T >= 0 && E >= 1 && k >= 1 && k <= E && d > 0 && d % 8 == 0, MOE4_EINVAL,
               "moe_router_wgrad: need 1 <= k <= E and d % 8 == 0");
  MOE4_REQUIRE(T * k < ((int64_t)1 << 31), MOE4_EINVAL, "moe_router_wgrad: T * k must be below 2^31");
  MOE4_REQUIRE(expert_off && dw && (T == 0 || (x && dlogits && perm)), MOE4_EINVAL, "moe_router_wgrad: NULL pointer");
  MOE4_REQUIRE(aligned16(x) && aligned16(dw), MOE4_EALIGN, "moe_router_wgrad: x and dw 16-byte aligned");
  const RwLayout L = rw_layout(T, E, k, d);
  MOE4_REQUIRE(ws != nullptr && ws_bytes >= (size_t)L.bytes, MOE4_EWORKSPACE,
               "moe_router_wgrad: workspace of moe_router_wgrad_ws_bytes() bytes required");
  MOE4_REQUIRE(aligned16(ws), MOE4_EALIGN, "moe_router_wgrad: ws 16-byte aligned");
  char* base = static_cast<char*>(ws);
  int32_t* coff = reinterpret_cast<int32_t*>(base);
  int32_t* chunk_e = reinterpret_cast<int32_t*>(base + L.off_chunk_e);
  float* part = reinterpret_cast<float*>(base + L.off_part);
  const hipStream_t s = as_stream(stream);
  hipLaunchKernelGGL(k_router_wgrad_chunks, dim3(1), dim3(rw::SCAN_T), 0, s, expert_off, E, T * k, L.bound, coff,
                     chunk_e);
  hipLaunchKernelGGL(k_router_wgrad_part, dim3((unsigned)L.bound, (unsigned)((d + rw::COLS - 1) / rw::COLS)),
                     dim3(rw::NT), 0, s, x, dlogits, perm, expert_off, coff, chunk_e, T, E, k, d, part);
  hipLaunchKernelGGL(k_router_wgrad_sum, dim3((unsigned)E, (unsigned)((d + rw::SUM_COLS - 1) / rw::SUM_COLS)),
                     dim3(rw::SUM_T), 0, s, coff, part, d, dw);
  return check_launch("moe_router_wgrad");
}
