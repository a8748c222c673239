// Host-side status reporting shared by every entry point.
#include "common.hpp"

#include <string>

namespace sdv {

namespace {
thread_local std::string g_last_error;
}

int32_t fail(int32_t code, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

void clear_error() { g_last_error.clear(); }

int32_t check_launch(const char *what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(SDV_E_HIP, "%s: %s", what, hipGetErrorString(e));
  return SDV_OK;
}

int num_cus() {
  static thread_local int cached_dev = -1;
  static thread_local int cached_cus = 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (dev != cached_dev) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      cus = 256;
    cached_dev = dev;
    cached_cus = cus;
  }
  return cached_cus;
}

}  // namespace sdv

extern "C" const char *sdv_last_error(void) { return sdv::g_last_error.c_str(); }

extern "C" int32_t sdv_version(void) { return 100; }
