// Internal helpers shared by the HIP sources of libmoe4 (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string>

#include "../../include/moe4.h"

namespace moe4 {

// ------------------------------------------------------------------ host side
void set_error(const std::string& msg);
int fail(int code, const std::string& msg);
int check_launch(const char* what);
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

#define MOE4_REQUIRE(cond, code, msg)                 \
  do {                                                \
    if (!(cond)) return ::moe4::fail((code), (msg));  \
  } while (0)

// Device-side error reports.  Each source file whose kernels can detect a
// problem on the device keeps a static __device__ error word of its own;
// kernels OR MOE4_DEVERR_* bits into it on their (rare) error paths, and
// moe4_debug_check() reads and clears each file's word through the readers
// below (synchronous copies, current device).
constexpr uint32_t MOE4_DEVERR_UNREADABLE = 0x80000000u;
uint32_t take_device_word(const void* symbol);  // read, then clear if non-zero
uint32_t take_dev_err_nvfp4();
uint32_t take_dev_err_route();
uint32_t take_dev_err_combine_q();
uint32_t take_dev_err_router();
// Test hook (moe4_debug_force_wait_timeout): bounded waits between
// workgroups wait for a count that never arrives, with a tiny spin limit, so
// that every wait gives up and reports MOE4_DEVERR_WAIT; kernels still exit.
bool force_wait_timeout();

// ---------------------------------------------------------------- device side
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// MurmurHash3 32-bit finaliser (A. Appleby, public domain), from its published
// description: xor-shift 16, multiply, xor-shift 13, multiply, xor-shift 16.
__host__ __device__ inline uint32_t fmix32(uint32_t h) {
  h ^= h >> 16;
  h *= 0x85EBCA6Bu;
  h ^= h >> 13;
  h *= 0xC2B2AE35u;
#if defined(__HIP_DEVICE_COMPILE__)
  // the product through an empty asm: otherwise the compiler turns a caller's
  // left shift of the result into a third (quarter-rate) 32-bit multiply
  asm("" : "+v"(h));
#endif
  h ^= h >> 16;
  return h;
}

// fmix32((x0 + p) ^ key) for p = 0..3, x0 % 4 == 0, with one first multiply
// for the four: x0 + p = x0 ^ p, the first xor-shift keeps that difference
// in the low two bits (h_p = h_0 ^ p), and (h ^ p) M = h M + ((t ^ p) - t) M
// modulo 2^32 with t = h & 3, where (t ^ 3) - t = ((t ^ 1) - t) + ((t ^ 2) - t).
// Made once per x0; word(p) finishes one of the four when it is needed.
struct Fmix32x4 {
  static constexpr uint32_t M1 = 0x85EBCA6Bu, M2 = 0xC2B2AE35u;
  uint32_t m0, d1, d2;
  __device__ Fmix32x4(uint32_t x0, uint32_t key) {
    uint32_t h = x0 ^ key;
    h ^= h >> 16;
    m0 = h * M1;
    // +-M1 and +-2 M1 as (c ^ s) - s with s = 0 or all ones (no select, whose
    // constant operands would each take a register)
    const uint32_t s1 = 0u - (h & 1u), s2 = 0u - ((h >> 1) & 1u);
    d1 = (M1 ^ s1) - s1;
    d2 = ((2u * M1) ^ s2) - s2;
  }
  __device__ uint32_t word(int p) const {
    uint32_t t = m0 + ((p & 1) ? d1 : 0u) + ((p & 2) ? d2 : 0u);
    t ^= t >> 13;
    t *= M2;
    asm("" : "+v"(t));  // (as in fmix32)
    return t ^ (t >> 16);
  }
};

// Seed/stream part of the stochastic-rounding key (host computes it once).
inline uint32_t sr_base_key(uint64_t seed, uint32_t stream_id) {
  uint32_t k = fmix32(static_cast<uint32_t>(seed));
  k = fmix32(k ^ static_cast<uint32_t>(seed >> 32));
  return fmix32(k ^ stream_id);  // the device applies fmix32(base ^ hi32(j))
}

__device__ inline float bf16_bits_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

// Round float32 to bf16 bits, ties to even (finite inputs).
__device__ inline uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Exact float32 value of an E4M3FN byte b < 256 (NaN codes never occur here):
// gfx950's FP8 converter decodes the OCP E4M3 format, and decodes all 254
// non-NaN bytes to the values of the field-by-field definition (exponent
// field e, mantissa m: (1 + m/8) 2^(e-7), subnormal m 2^-9), one instruction.
__device__ inline float e4m3_to_f32(uint32_t b) { return __builtin_amdgcn_cvt_f32_fp8((int)b, 0); }

// Mantissa factor 1.m of a positive normal float (its value over 2**floor(log2)).
__device__ inline float mant_factor(float s) {
  return __uint_as_float((__float_as_uint(s) & 0x007FFFFFu) | 0x3F800000u);
}

// Cross-lane moves without LDS: DPP within each row of 16 lanes, and the
// permlane swaps between rows (each returns the value of lane l and of lane
// l ^ 16, or l ^ 32, in its two results).
template <int CTRL>
__device__ inline uint32_t dpp_u(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
constexpr int DPP_XOR1 = 0xB1;         // quad_perm [1, 0, 3, 2]: lane l ^ 1
constexpr int DPP_XOR2 = 0x4E;         // quad_perm [2, 3, 0, 1]: lane l ^ 2
constexpr int DPP_HALF_MIRROR = 0x141;  // lane 7 - l within each 8
constexpr int DPP_XOR8 = 0x128;         // row_ror 8: lane l ^ 8 within each 16
__device__ inline float lane_xor1(float v) { return __uint_as_float(dpp_u<DPP_XOR1>(__float_as_uint(v))); }
__device__ inline float lane_xor2(float v) { return __uint_as_float(dpp_u<DPP_XOR2>(__float_as_uint(v))); }
__device__ inline float lane_xor8(float v) { return __uint_as_float(dpp_u<DPP_XOR8>(__float_as_uint(v))); }
// max of the values of lanes l and l ^ 16 / l ^ 32
__device__ inline float max_xor16(float v) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ inline float max_xor32(float v) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ inline uint32_t umax_xor16(uint32_t v) {
  const auto p = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return max((uint32_t)p[0], (uint32_t)p[1]);
}
__device__ inline uint32_t umax_xor32(uint32_t v) {
  const auto p = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return max((uint32_t)p[0], (uint32_t)p[1]);
}

// Wave-wide reductions (wave64): the maximum in every lane (each step pairs the two halves of a
// group of lanes: 2, 4, 8, 16, 32, 64).
__device__ inline float wave_max(float v) {
  v = fmaxf(v, lane_xor1(v));
  v = fmaxf(v, lane_xor2(v));
  v = fmaxf(v, __uint_as_float(dpp_u<DPP_HALF_MIRROR>(__float_as_uint(v))));
  v = fmaxf(v, lane_xor8(v));
  v = max_xor16(v);
  return max_xor32(v);
}
__device__ inline uint32_t wave_umax(uint32_t v) {
  v = max(v, dpp_u<DPP_XOR1>(v));
  v = max(v, dpp_u<DPP_XOR2>(v));
  v = max(v, dpp_u<DPP_HALF_MIRROR>(v));
  v = max(v, dpp_u<DPP_XOR8>(v));
  v = umax_xor16(v);
  return umax_xor32(v);
}

}  // namespace moe4
