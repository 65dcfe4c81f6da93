// Host-side plumbing of libmoe4: error reporting, version, the constant
// activation tables and the device-side error words.
#include <atomic>
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

// The SiLU (g_act_tab[0]) and SiLU' (g_act_tab[1]) tables: initialised data
// of the code object, written at build time by gen_act_tab.cpp (correctly
// rounded float32 values for |u| in [2**-16, 2**8)) and never written at run
// time.  Nothing fills them, so no call waits for a table and any call may be
// captured in a graph.  (Not declared const: a const namespace-scope variable
// has internal linkage, and the runtime's symbol lookup cannot find it.)
__device__ float g_act_tab[2][ACT_TAB] = {
#include "act_tab.inc"
};

static std::mutex g_act_mu;
static const float* g_act_ptr[64];

int act_tables(const float** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return fail(MOE4_EHIP, "hipGetDevice failed");
  std::lock_guard<std::mutex> lock(g_act_mu);
  if (g_act_ptr[dev] == nullptr) {
    // the device address of the constant table (a query: no stream work)
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(g_act_tab)) != hipSuccess || p == nullptr)
      return fail(MOE4_EHIP, "hipGetSymbolAddress(g_act_tab) failed");
    g_act_ptr[dev] = static_cast<const float*>(p);
  }
  *out = g_act_ptr[dev];
  return MOE4_OK;
}

// ---------------------------------------------------- device-side error words

static std::atomic<int> g_force_wait_timeout{0};

bool force_wait_timeout() { return g_force_wait_timeout.load(std::memory_order_relaxed) != 0; }

uint32_t take_device_word(const void* symbol) {
  uint32_t v = 0;
  if (hipMemcpyFromSymbol(&v, symbol, sizeof v, 0, hipMemcpyDeviceToHost) != hipSuccess) return MOE4_DEVERR_UNREADABLE;
  if (v != 0) {
    const uint32_t z = 0;
    if (hipMemcpyToSymbol(symbol, &z, sizeof z, 0, hipMemcpyHostToDevice) != hipSuccess) v |= MOE4_DEVERR_UNREADABLE;
  }
  return v;
}

}  // namespace moe4

extern "C" const char* moe4_last_error(void) { return moe4::t_last_error.c_str(); }
extern "C" const char* moe4_version(void) { return "moe4 0.2 gfx950"; }

extern "C" int moe4_debug_check(void* stream) {
  using namespace moe4;
  hipError_t e = hipStreamSynchronize(as_stream(stream));
  if (e == hipSuccess) e = hipGetLastError();
  if (e != hipSuccess) return fail(MOE4_EHIP, std::string("moe4_debug_check: ") + hipGetErrorString(e));
  const uint32_t bits = take_dev_err_nvfp4() | take_dev_err_route() | take_dev_err_combine_q() | take_dev_err_router();
  if (bits == 0) return MOE4_OK;
  std::string msg = "moe4_debug_check: device-side error";
  if (bits & MOE4_DEVERR_WAIT) msg += "; a bounded wait between workgroups gave up (that call's results are wrong)";
  if (bits & MOE4_DEVERR_INDEX) msg += "; an index or offset outside its range was clamped";
  if (bits & MOE4_DEVERR_UNREADABLE) msg += "; a device error word could not be read or cleared";
  return fail(MOE4_EDEVICE, msg);
}

extern "C" int moe4_debug_force_wait_timeout(int on) {
  moe4::g_force_wait_timeout.store(on ? 1 : 0, std::memory_order_relaxed);
  return MOE4_OK;
}
