// Host-side plumbing of libmoe4: error reporting, version, and the one-time
// activation tables.
#include <mutex>
#include <string>

#include "act.h"
#include "moe4_internal.h"

namespace moe4 {

static thread_local std::string t_last_error;

void set_error(const std::string& msg) { t_last_error = msg; }

int fail(int code, const std::string& msg) {
  t_last_error = msg;
  return code;
}

int check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(MOE4_EHIP, std::string(what) + ": " + hipGetErrorString(e));
  return MOE4_OK;
}

__device__ float g_act_tab[2][ACT_TAB];

__global__ void k_fill_act_tables(float* tab) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= ACT_TAB) return;
  // index -> bf16 pattern: sign (bit 11), binade (bits 7..10), mantissa (0..6)
  uint32_t s = (uint32_t)i >> 11, ex = (((uint32_t)i >> 7) & 15u) + 119u, m = (uint32_t)i & 0x7Fu;
  uint32_t b = (s << 15) | (ex << 7) | m;
  double x = (double)bf16_bits_to_f32(b);
  tab[i] = (float)silu_f64(x);
  tab[ACT_TAB + i] = (float)dsilu_f64(x);
}

static std::mutex g_act_mu;
static const float* g_act_ptr[64];
static bool g_act_done[64];

int ensure_act_tables(hipStream_t s) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return fail(MOE4_EHIP, "hipGetDevice failed");
  std::lock_guard<std::mutex> lock(g_act_mu);
  if (g_act_done[dev]) return MOE4_OK;
  void* p = nullptr;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(g_act_tab)) != hipSuccess || p == nullptr)
    return fail(MOE4_EHIP, "hipGetSymbolAddress(g_act_tab) failed");
  g_act_ptr[dev] = static_cast<const float*>(p);
  hipLaunchKernelGGL(k_fill_act_tables, dim3((ACT_TAB + 255) / 256), dim3(256), 0, s, static_cast<float*>(p));
  int rc = check_launch("k_fill_act_tables");
  if (rc) return rc;
  // one-time: wait, so that later calls on any stream see the filled table
  if (hipStreamSynchronize(s) != hipSuccess) return fail(MOE4_EHIP, "activation table fill failed");
  g_act_done[dev] = true;
  return MOE4_OK;
}

const float* act_tables_device_ptr() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lock(g_act_mu);
  return g_act_ptr[dev];
}

}  // namespace moe4

extern "C" const char* moe4_last_error(void) { return moe4::t_last_error.c_str(); }
extern "C" const char* moe4_version(void) { return "moe4 0.1 gfx950"; }

extern "C" int moe4_debug_check(void* stream) {
  hipError_t e = hipStreamSynchronize(static_cast<hipStream_t>(stream));
  if (e == hipSuccess) e = hipGetLastError();
  if (e != hipSuccess) return moe4::fail(MOE4_EHIP, std::string("moe4_debug_check: ") + hipGetErrorString(e));
  return MOE4_OK;
}
