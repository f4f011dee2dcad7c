// Library-wide C-ABI glue: thread-local error messages, launch checks, version.
#include "moe_internal.h"

#include <mutex>
#include <vector>

namespace moeffn {

static thread_local std::string g_last_error;

void set_error(const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
}

void clear_error() { g_last_error.clear(); }

moe_status check_launch(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("%s: %s", what, hipGetErrorString(e));
    return MOE_EHIP;
  }
  return MOE_OK;
}

int device_cu_count() {
  static std::mutex mu;
  static std::vector<int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  std::lock_guard<std::mutex> lock(mu);
  if ((int)cache.size() <= dev) cache.resize(dev + 1, 0);
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

}  // namespace moeffn

extern "C" const char* moe_last_error(void) { return moeffn::g_last_error.c_str(); }
extern "C" const char* moe_version(void) { return "moeffn 0.1 (gfx950)"; }
