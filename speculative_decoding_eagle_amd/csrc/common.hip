// Host-side status reporting shared by every entry point.
#include "common.hpp"

#include <atomic>
#include <string>

namespace sdv {

namespace {
thread_local std::string g_last_error;
constexpr uint32_t kLibraryDefault = 0xFFFFFFFFu;
std::atomic<uint32_t> g_wait_limit{kLibraryDefault};

__global__ void zero_words_kernel(unsigned *p, size_t n) {
  const size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}
}  // namespace

unsigned wait_limit(unsigned dflt) {
  const uint32_t v = g_wait_limit.load(std::memory_order_relaxed);
  return v == kLibraryDefault ? dflt : v;
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

extern "C" int32_t sdv_version(void) { return 101; }

extern "C" uint32_t sdv_set_wait_limit(uint32_t polls) {
  return sdv::g_wait_limit.exchange(polls, std::memory_order_relaxed);
}

extern "C" int32_t sdv_workspace_status(void *ws, size_t ws_bytes, uint32_t *status, int32_t reset, void *stream) {
  using namespace sdv;
  clear_error();
  SDV_REQUIRE(status, SDV_E_NULL, "workspace_status: NULL status pointer");
  *status = 0;
  if (!ws || ws_bytes < kWsHeaderBytes) return SDV_OK;
  hipStream_t st = as_stream(stream);
  uint32_t word = 0;
  hipError_t e = hipMemcpyAsync(&word, ws, sizeof(word), hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return fail(SDV_E_HIP, "workspace_status: %s", hipGetErrorString(e));
  *status = word;
  if (reset && word != 0) {
    const size_t n = ws_bytes / sizeof(unsigned);
    hipLaunchKernelGGL(zero_words_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, st,
                       static_cast<unsigned *>(ws), n);
    const int32_t rc = check_launch("workspace_status: reset");
    if (rc != SDV_OK) return rc;
  }
  return SDV_OK;
}

extern "C" int32_t sdv_tli_check(int32_t topk, int32_t num_steps, int32_t num_draft_tokens) {
  using namespace sdv;
  clear_error();
  SDV_REQUIRE(topk == 1, SDV_E_UNSUPPORTED, "tli_check: TLI drafts one candidate per step (topk=%d, need 1)", topk);
  SDV_REQUIRE(num_steps >= 1 && num_draft_tokens == num_steps + 1, SDV_E_UNSUPPORTED,
              "tli_check: TLI needs num_draft_tokens == num_steps + 1 (got %d and %d)", num_draft_tokens, num_steps);
  return SDV_OK;
}
