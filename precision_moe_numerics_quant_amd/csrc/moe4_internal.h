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
  h ^= h >> 16;
  return h;
}

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

// Wave-wide reductions (wave64).
__device__ inline float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ inline uint32_t wave_umax(uint32_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o, 64));
  return v;
}

}  // namespace moe4
