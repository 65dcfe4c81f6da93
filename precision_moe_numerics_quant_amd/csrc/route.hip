// Routing and data movement around the expert GEMMs (gfx950): top-k with
// renormalised gates, the deterministic stable permutation of assignments
// into expert order, the NVFP4 row gather (the single-GPU stand-in for the
// pages' NVFP4 dispatch, lhc.media page, paragraph on communication), the
// gate-weighted combine and the un-permuting sum of the backward pass.
//
// The permutation is a counting sort without order-dependent atomics: tokens
// are cut into chunks of 64 (one wave); per chunk an LDS bit mask per expert
// records which lanes chose it, so a lane's rank among the chunk's
// assignments to that expert is a popcount; a per-expert scan over chunks
// then gives each chunk's base row.  The result is the stable order (expert
// ascending, token ascending) on every run.
#include "moe4_internal.h"

namespace moe4 {

// This file's device-side error word (moe4_debug_check reads and clears it):
// indices or offsets outside their range, clamped so that nothing faults.
static __device__ uint32_t g_dev_err;
uint32_t take_dev_err_route() { return take_device_word(&g_dev_err); }

// idx clamped to [0, n); a clamp is reported
__device__ inline int64_t clamp_index(int64_t i, int64_t n) {
  if (i < 0 || i >= n) {
    atomicOr(&g_dev_err, MOE4_DEVERR_INDEX);
    return i < 0 ? 0 : n - 1;
  }
  return i;
}

constexpr int MAXE = 1024;
constexpr int MAXK = 16;

// ------------------------------------------------------------------- top-k
__global__ void __launch_bounds__(256) k_topk(const float* __restrict__ logits, const float* __restrict__ bias,
                                              int64_t T, int E, int k, int32_t* __restrict__ idx,
                                              float* __restrict__ gates) {
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= T) return;
  constexpr int PER = MAXE / 64;
  float z[PER];
  bool taken[PER];
#pragma unroll
  for (int s = 0; s < PER; ++s) {
    const int e = lane + 64 * s;
    taken[s] = e >= E;
    float v = 0.0f;
    if (e < E) {
      v = logits[t * E + e];
      if (bias) v = v + bias[e];
    }
    z[s] = v;
  }
  float zsel[MAXK];
  for (int j = 0; j < k; ++j) {
    float bv = 0.0f;
    int be = 0x7FFFFFFF;
#pragma unroll
    for (int s = 0; s < PER; ++s) {
      const int e = lane + 64 * s;
      if (!taken[s] && (be == 0x7FFFFFFF || z[s] > bv)) { bv = z[s]; be = e; }
    }
    // wave arg-max: larger value wins, equal values -> lower expert index
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      float ov = __shfl_xor(bv, o, 64);
      int oe = __shfl_xor(be, o, 64);
      bool take = (oe != 0x7FFFFFFF) && (be == 0x7FFFFFFF || ov > bv || (ov == bv && oe < be));
      if (take) { bv = ov; be = oe; }
    }
#pragma unroll
    for (int s = 0; s < PER; ++s)
      if (lane + 64 * s == be) taken[s] = true;
    zsel[j] = bv;
    if (lane == 0) idx[t * k + j] = be;
  }
  if (lane < k) {
    float s = 0.0f;
    float wj = 0.0f;
    for (int j = 0; j < k; ++j) {
      float w = (float)exp((double)(zsel[j] - zsel[0]));
      s = s + w;
      if (j == lane) wj = w;
    }
    gates[t * k + lane] = wj / s;
  }
}

// ------------------------------------------------------------- permutation
__global__ void __launch_bounds__(64) k_route_hist(const int32_t* __restrict__ idx, int64_t T, int E, int k,
                                                   uint32_t* __restrict__ cnt, uint8_t* __restrict__ rank) {
  __shared__ unsigned long long mask[MAXE];
  const int lane = threadIdx.x;
  const int64_t chunk = blockIdx.x;
  for (int e = lane; e < E; e += 64) mask[e] = 0ull;
  __syncthreads();
  const int64_t t = chunk * 64 + lane;
  if (t < T)
    for (int j = 0; j < k; ++j) {
      int e = idx[t * k + j];
      e = e < 0 ? 0 : (e >= E ? E - 1 : e);
      atomicOr(&mask[e], 1ull << lane);
    }
  __syncthreads();
  if (t < T) {
    const unsigned long long below = (1ull << lane) - 1ull;
    for (int j = 0; j < k; ++j) {
      int e = idx[t * k + j];
      e = e < 0 ? 0 : (e >= E ? E - 1 : e);
      rank[t * k + j] = (uint8_t)__popcll(mask[e] & below);
    }
  }
  for (int e = lane; e < E; e += 64) cnt[chunk * E + e] = (uint32_t)__popcll(mask[e]);
}

__global__ void __launch_bounds__(MAXE) k_route_scan(uint32_t* __restrict__ cnt, int64_t n_chunks, int E,
                                                     int32_t* __restrict__ off, int32_t* __restrict__ off_pad) {
  __shared__ uint32_t tot[MAXE];
  const int e = threadIdx.x;
  if (e < E) {
    uint32_t run = 0;
    for (int64_t c = 0; c < n_chunks; ++c) {
      uint32_t v = cnt[c * E + e];
      cnt[c * E + e] = run;  // becomes the chunk's base within expert e
      run += v;
    }
    tot[e] = run;
  }
  __syncthreads();
  if (e == 0) {
    int32_t o = 0, op = 0;
    for (int i = 0; i < E; ++i) {
      off[i] = o;
      off_pad[i] = op;
      o += (int32_t)tot[i];
      op += (int32_t)((tot[i] + 31u) / 32u * 32u);
    }
    off[E] = o;
    off_pad[E] = op;
  }
}

__global__ void k_route_scatter(const int32_t* __restrict__ idx, int64_t A, int E, int k,
                                const uint32_t* __restrict__ base, const uint8_t* __restrict__ rank,
                                const int32_t* __restrict__ off, int32_t* __restrict__ perm,
                                int32_t* __restrict__ inv_perm) {
  const int64_t a = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (a >= A) return;
  int e = idx[a];
  e = e < 0 ? 0 : (e >= E ? E - 1 : e);
  const int64_t chunk = (a / k) / 64;
  int64_t row = (int64_t)off[e] + base[chunk * E + e] + rank[a];
  row = row < 0 ? 0 : (row >= A ? A - 1 : row);
  perm[row] = (int32_t)a;
  inv_perm[a] = (int32_t)row;
}

// ------------------------------------------------------------------ gather
__global__ void __launch_bounds__(256) k_gather_rows(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ sf,
                                                     int64_t n_in, int64_t cols, const int32_t* __restrict__ perm,
                                                     int k, uint8_t* __restrict__ oc, uint8_t* __restrict__ os) {
  const int64_t r = blockIdx.x;
  const int64_t a = perm[r];
  const int64_t src = clamp_index(a < 0 ? -1 : a / k, n_in);
  const int64_t cb = cols / 2;  // multiple of 8
  const u32x2* s2 = reinterpret_cast<const u32x2*>(codes + src * cb);
  u32x2* d2 = reinterpret_cast<u32x2*>(oc + r * cb);
  for (int64_t i = threadIdx.x; i < cb / 8; i += 256) d2[i] = s2[i];
  const int64_t sb = cols / 16;
  for (int64_t i = threadIdx.x; i < sb; i += 256) os[r * sb + i] = sf[src * sb + i];
}

// --------------------------------------------------------- combine / unpermute
template <bool GATED>
__global__ void __launch_bounds__(256) k_combine(const float* __restrict__ yp, const float* __restrict__ gates,
                                                 const int32_t* __restrict__ inv, int64_t T, int k, int64_t d,
                                                 int64_t n_rows, uint16_t* __restrict__ y) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;  // one quad of columns
  const int64_t nq = d / 4;
  if (q >= T * nq) return;
  const int64_t t = q / nq, c = (q % nq) * 4;
  // all k row indices, then all k row loads in flight, then the sum in slot
  // order (k <= MAXK, checked at launch)
  int64_t rows[MAXK];
  float g[MAXK];
#pragma unroll
  for (int j = 0; j < MAXK; ++j) {
    if (j < k) {
      rows[j] = clamp_index(inv[t * k + j], n_rows);
      g[j] = GATED ? gates[t * k + j] : 1.0f;
    }
  }
  f32x4 v[MAXK];
#pragma unroll
  for (int j = 0; j < MAXK; ++j)
    if (j < k) v[j] = *reinterpret_cast<const f32x4*>(yp + rows[j] * d + c);
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int j = 0; j < MAXK; ++j) {
    if (j < k) {
      if (GATED) {
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = acc[i] + g[j] * v[j][i];
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = acc[i] + v[j][i];
      }
    }
  }
  u32x2 out = {f32_to_bf16_bits(acc[0]) | (f32_to_bf16_bits(acc[1]) << 16),
               f32_to_bf16_bits(acc[2]) | (f32_to_bf16_bits(acc[3]) << 16)};
  *reinterpret_cast<u32x2*>(y + t * d + c) = out;
}

// Gate gradient: dg[t, j] = sum_c dy[t, c] * yp[inv[t*k + j], c], one wave per
// token.  Lane l takes columns 8 l + 512 i (16-byte bf16 loads of dy, two
// 16-byte loads of yp), accumulates in float32 in column order, then the
// wave sums the 64 lane totals in a fixed butterfly order (deterministic).
__global__ void __launch_bounds__(256) k_dgates(const uint16_t* __restrict__ dy, const float* __restrict__ yp,
                                                const int32_t* __restrict__ inv, int64_t T, int k, int64_t d,
                                                int64_t n_rows, float* __restrict__ dg) {
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int l = threadIdx.x & 63;
  if (t >= T) return;
  const uint16_t* dyr = dy + t * d;
  // the token's dy row is read once (kept in registers up to d = 8192) for all
  // k slots; each lane sums its columns 8 l + 512 i in order either way
  constexpr int DYC = 16;
  u32x4 dyc[DYC];
  const bool cached = d <= 512 * DYC;
  if (cached) {
#pragma unroll
    for (int i = 0; i < DYC; ++i) {
      const int64_t c = 8 * l + 512 * i;
      dyc[i] = c < d ? *reinterpret_cast<const u32x4*>(dyr + c) : u32x4{0u, 0u, 0u, 0u};
    }
  }
  auto add8 = [](float acc, const u32x4 g, const f32x4 a, const f32x4 b) {
    acc = acc + bf16_bits_to_f32(g[0] & 0xFFFFu) * a[0];
    acc = acc + bf16_bits_to_f32(g[0] >> 16) * a[1];
    acc = acc + bf16_bits_to_f32(g[1] & 0xFFFFu) * a[2];
    acc = acc + bf16_bits_to_f32(g[1] >> 16) * a[3];
    acc = acc + bf16_bits_to_f32(g[2] & 0xFFFFu) * b[0];
    acc = acc + bf16_bits_to_f32(g[2] >> 16) * b[1];
    acc = acc + bf16_bits_to_f32(g[3] & 0xFFFFu) * b[2];
    acc = acc + bf16_bits_to_f32(g[3] >> 16) * b[3];
    return acc;
  };
  for (int j = 0; j < k; ++j) {
    const int64_t row = clamp_index(inv[t * k + j], n_rows);
    const float* ypr = yp + row * d;
    float acc = 0.0f;
    if (cached) {
#pragma unroll
      for (int i = 0; i < DYC; ++i) {
        const int64_t c = 8 * l + 512 * i;
        if (c < d)
          acc = add8(acc, dyc[i], *reinterpret_cast<const f32x4*>(ypr + c), *reinterpret_cast<const f32x4*>(ypr + c + 4));
      }
    } else {
      for (int64_t c = 8 * l; c < d; c += 512)
        acc = add8(acc, *reinterpret_cast<const u32x4*>(dyr + c), *reinterpret_cast<const f32x4*>(ypr + c),
                   *reinterpret_cast<const f32x4*>(ypr + c + 4));
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) acc = acc + __shfl_xor(acc, o, 64);
    if (l == 0) dg[t * k + j] = acc;
  }
}

// Router backward: the gates are a softmax of z over the selected experts,
// so dz[t, e_j] = g_j * (dg_j - s), s = sum_i g_i * dg_i (float32, in slot
// order, no fused multiply-add), and 0 for the experts not selected.  One
// wave per token; lane l writes experts l, l + 64, ... (one store each).
__global__ void __launch_bounds__(256) k_route_backward(const float* __restrict__ dg, const float* __restrict__ gates,
                                                        const int32_t* __restrict__ idx, int64_t T, int E, int k,
                                                        float* __restrict__ dz) {
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int l = threadIdx.x & 63;
  if (t >= T) return;
  const float* g = gates + t * k;
  const float* d = dg + t * k;
  const int32_t* ix = idx + t * k;
  float s = 0.0f;
  for (int i = 0; i < k; ++i) s = s + g[i] * d[i];
  for (int e = l; e < E; e += 64) {
    float v = 0.0f;
    for (int j = 0; j < k; ++j)
      if (ix[j] == e) v = g[j] * (d[j] - s);
    dz[t * E + e] = v;
  }
}

}  // namespace moe4

using namespace moe4;

static int64_t route_chunks(int64_t T) { return (T + 63) / 64; }

extern "C" size_t moe_route_topk_ws_bytes(int64_t T, int32_t E, int32_t k) {
  const int64_t cnt = route_chunks(T) * (int64_t)E * 4;
  const int64_t rk = T * (int64_t)k;
  return (size_t)(((cnt + 15) / 16) * 16 + ((rk + 15) / 16) * 16 + 16);
}

extern "C" int moe_route_topk(const float* logits, const float* bias, int64_t T, int32_t E, int32_t k,
                              int32_t* topk_idx, float* gates, int32_t* expert_off, int32_t* expert_off_pad,
                              int32_t* perm, int32_t* inv_perm, void* ws, size_t ws_bytes, void* stream) {
  MOE4_REQUIRE(T >= 0 && E >= 1 && E <= MAXE && k >= 1 && k <= MAXK && k <= E, MOE4_EINVAL,
               "moe_route_topk: need T >= 0, 1 <= k <= min(E, 16), E <= 1024");
  MOE4_REQUIRE(T * (int64_t)k < ((int64_t)1 << 31), MOE4_EINVAL, "moe_route_topk: T*k must fit int32");
  MOE4_REQUIRE(expert_off && expert_off_pad && ws, MOE4_EINVAL, "moe_route_topk: NULL pointer");
  MOE4_REQUIRE(T == 0 || (logits && topk_idx && gates && perm && inv_perm), MOE4_EINVAL, "moe_route_topk: NULL pointer");
  MOE4_REQUIRE(ws_bytes >= moe_route_topk_ws_bytes(T, E, k), MOE4_EWORKSPACE, "moe_route_topk: workspace too small");
  MOE4_REQUIRE(aligned16(ws), MOE4_EALIGN, "moe_route_topk: workspace must be 16-byte aligned");
  hipStream_t s = as_stream(stream);
  const int64_t nch = route_chunks(T);
  uint32_t* cnt = static_cast<uint32_t*>(ws);
  uint8_t* rank = static_cast<uint8_t*>(ws) + ((nch * E * 4 + 15) / 16) * 16;
  if (T > 0) {
    hipLaunchKernelGGL(k_topk, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, s, logits, bias, T, E, k, topk_idx, gates);
    hipLaunchKernelGGL(k_route_hist, dim3((unsigned)nch), dim3(64), 0, s, topk_idx, T, E, k, cnt, rank);
  }
  hipLaunchKernelGGL(k_route_scan, dim3(1), dim3(MAXE), 0, s, cnt, nch, E, expert_off, expert_off_pad);
  if (T > 0) {
    const int64_t A = T * k;
    hipLaunchKernelGGL(k_route_scatter, dim3((unsigned)((A + 255) / 256)), dim3(256), 0, s, topk_idx, A, E, k, cnt,
                       rank, expert_off, perm, inv_perm);
  }
  return check_launch("moe_route_topk");
}

extern "C" int moe_gather_rows(const uint8_t* codes, const uint8_t* sf, int64_t n_rows_in, int64_t cols,
                               const int32_t* perm, int32_t k, int64_t n_rows_out, uint8_t* out_codes,
                               uint8_t* out_sf, void* stream) {
  MOE4_REQUIRE(cols > 0 && cols % 16 == 0 && k >= 1 && n_rows_in >= 0 && n_rows_out >= 0, MOE4_EINVAL,
               "moe_gather_rows: bad sizes");
  MOE4_REQUIRE(n_rows_out == 0 || (n_rows_in > 0 && codes && sf && perm && out_codes && out_sf), MOE4_EINVAL,
               "moe_gather_rows: NULL pointer");
  MOE4_REQUIRE(aligned16(codes) && aligned16(out_codes), MOE4_EALIGN, "moe_gather_rows: misaligned pointer");
  MOE4_REQUIRE(n_rows_out < ((int64_t)1 << 31), MOE4_EINVAL, "moe_gather_rows: too many rows");
  if (n_rows_out == 0) return MOE4_OK;
  hipLaunchKernelGGL(k_gather_rows, dim3((unsigned)n_rows_out), dim3(256), 0, as_stream(stream), codes, sf, n_rows_in,
                     cols, perm, k, out_codes, out_sf);
  return check_launch("moe_gather_rows");
}

extern "C" int moe_combine(const float* yp, const float* gates, const int32_t* inv_perm, int64_t T, int32_t k,
                           int64_t d, uint16_t* y, void* stream) {
  MOE4_REQUIRE(T >= 0 && k >= 1 && k <= MAXK && d > 0 && d % 4 == 0, MOE4_EINVAL,
               "moe_combine: bad sizes (1 <= k <= 16, d % 4 == 0)");
  MOE4_REQUIRE(T == 0 || (yp && gates && inv_perm && y), MOE4_EINVAL, "moe_combine: NULL pointer");
  MOE4_REQUIRE(aligned16(yp) && aligned16(y), MOE4_EALIGN, "moe_combine: misaligned pointer");
  if (T == 0) return MOE4_OK;
  const int64_t n = T * (d / 4);
  hipLaunchKernelGGL((k_combine<true>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0, as_stream(stream), yp, gates,
                     inv_perm, T, k, d, T * k, y);
  return check_launch("moe_combine");
}

extern "C" int moe_unpermute_sum(const float* dxp, const int32_t* inv_perm, int64_t T, int32_t k, int64_t d,
                                 uint16_t* dx, void* stream) {
  MOE4_REQUIRE(T >= 0 && k >= 1 && k <= MAXK && d > 0 && d % 4 == 0, MOE4_EINVAL,
               "moe_unpermute_sum: bad sizes (1 <= k <= 16, d % 4 == 0)");
  MOE4_REQUIRE(T == 0 || (dxp && inv_perm && dx), MOE4_EINVAL, "moe_unpermute_sum: NULL pointer");
  MOE4_REQUIRE(aligned16(dxp) && aligned16(dx), MOE4_EALIGN, "moe_unpermute_sum: misaligned pointer");
  if (T == 0) return MOE4_OK;
  const int64_t n = T * (d / 4);
  hipLaunchKernelGGL((k_combine<false>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0, as_stream(stream), dxp,
                     nullptr, inv_perm, T, k, d, T * k, dx);
  return check_launch("moe_unpermute_sum");
}

extern "C" int moe_dgates(const uint16_t* dy, const float* yp, const int32_t* inv_perm, int64_t T, int32_t k,
                          int64_t d, float* dg, void* stream) {
  MOE4_REQUIRE(T >= 0 && k >= 1 && k <= MAXK && d > 0 && d % 8 == 0, MOE4_EINVAL,
               "moe_dgates: bad sizes (1 <= k <= 16, d % 8 == 0)");
  MOE4_REQUIRE(T == 0 || (dy && yp && inv_perm && dg), MOE4_EINVAL, "moe_dgates: NULL pointer");
  MOE4_REQUIRE(aligned16(dy) && aligned16(yp), MOE4_EALIGN, "moe_dgates: misaligned pointer");
  if (T == 0) return MOE4_OK;
  hipLaunchKernelGGL(k_dgates, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, as_stream(stream), dy, yp, inv_perm, T, k,
                     d, T * k, dg);
  return check_launch("moe_dgates");
}

extern "C" int moe_route_backward(const float* dg, const float* gates, const int32_t* topk_idx, int64_t T, int32_t E,
                                  int32_t k, float* dlogits, void* stream) {
  MOE4_REQUIRE(T >= 0 && E >= 1 && k >= 1 && k <= MAXK && k <= E, MOE4_EINVAL,
               "moe_route_backward: need T >= 0, 1 <= k <= min(E, 16)");
  MOE4_REQUIRE(T == 0 || (dg && gates && topk_idx && dlogits), MOE4_EINVAL, "moe_route_backward: NULL pointer");
  if (T == 0) return MOE4_OK;
  hipLaunchKernelGGL(k_route_backward, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, as_stream(stream), dg, gates,
                     topk_idx, T, E, k, dlogits);
  return check_launch("moe_route_backward");
}
