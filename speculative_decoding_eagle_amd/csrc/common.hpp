// Shared host/device helpers of the gfx950 library: status reporting, launch
// checks, workspace carving and a few wave-level primitives.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstddef>
#include <cstdint>
#include <cstdio>

#include "../../include/sdv.h"

namespace sdv {

// ---------------------------------------------------------------- host side

// Records `msg` as the calling thread's last error and returns `code`.
int32_t fail(int32_t code, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

// Checks the launch that was just enqueued.
int32_t check_launch(const char *what);

inline hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Carves consecutive 256-byte aligned regions out of a caller workspace.
struct Carver {
  char *base;
  size_t used = 0;
  explicit Carver(void *p) : base(static_cast<char *>(p)) {}
  template <typename T>
  T *take(size_t count) {
    used = align_up(used, 256);
    T *p = base ? reinterpret_cast<T *>(base + used) : nullptr;
    used += count * sizeof(T);
    return p;
  }
  size_t bytes() const { return align_up(used, 256); }
};

// Number of compute units of the current device (cached per device).
int num_cus();

// Workspaces whose kernels wait on one another begin with a 256-byte header;
// word 0 is the sticky status word (SDV_STATUS_* bits) that
// sdv_workspace_status reads.  The TLI scatter keeps the (K, V_target) of the
// call that built its inverse in words 1-3.
constexpr size_t kWsHeaderBytes = 256;
constexpr int kWsStatus = 0;
constexpr int kWsTliK = 1, kWsTliV = 2, kWsTliMagic = 3;
constexpr unsigned kTliMagic = 0x544C4931u;
inline unsigned *ws_header(void *ws) { return static_cast<unsigned *>(ws); }

// Polls a bounded wait makes before it gives up: `dflt` unless a test set a
// limit with sdv_set_wait_limit (0: give up at once, without polling).
unsigned wait_limit(unsigned dflt);

// The K and V pools of every layer, passed to a kernel by value.
constexpr int kMaxLayers = 128;
struct PoolPtrs {
  uint16_t *k[kMaxLayers];
  uint16_t *v[kMaxLayers];
};

#define SDV_REQUIRE(cond, code, ...)          \
  do {                                        \
    if (!(cond)) return ::sdv::fail((code), __VA_ARGS__); \
  } while (0)

// ---------------------------------------------------------------- device side

constexpr int kWave = 64;

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// IEEE-754-2019 maximum (NaN propagates): one v_maximum3_f32 on gfx950,
// with no NaN-quieting of its inputs in front of it as fmaxf needs.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// Strict total order used by every top-k / argmax: larger value first, then
// lower index.
__device__ __forceinline__ bool better(float v, int i, float w, int j) {
  return v > w || (v == w && i < j);
}

// Wave-wide reduction to the best (value, index) pair; every lane gets it.
__device__ __forceinline__ void wave_best(float &v, int &i) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    float ov = __shfl_xor(v, off, kWave);
    int oi = __shfl_xor(i, off, kWave);
    if (better(ov, oi, v, i)) {
      v = ov;
      i = oi;
    }
  }
}

// Sets status bits in a workspace header (device scope, relaxed: the word
// is read by the host after the stream has drained).
__device__ __forceinline__ void raise_status(unsigned *status, unsigned bits) {
  __hip_atomic_fetch_or(status, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ unsigned long long wave_sum_u64(unsigned long long x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, kWave);
  return x;
}

// ------------------------------------------------------------ LDS DMA

// 16 bytes per lane from global memory straight into LDS: lane L writes LDS
// bytes lds_addr + 16*L .. +15 (lds_addr is wave-uniform, via M0).  Issued
// as inline assembly so that the compiler does not add its conservative
// "wait for every LDS DMA before any LDS read"; the kernels wait explicitly
// (wait_vmcnt) and the memory clobber keeps LDS reads from moving across.
__device__ __forceinline__ void dma16(const void *gaddr, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(gaddr), "s"(lds_addr) : "memory", "m0");
}

// As dma16, addressed as a 64-bit base in scalar registers plus this
// lane's 32-bit byte offset.
__device__ __forceinline__ void dma16s(uint32_t voff, const void *sbase, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(voff), "s"(sbase), "s"(lds_addr)
               : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_offset(const void *p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p));   // low half of the flat address
}

// s_waitcnt with only the vector-memory counter bounded (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

}  // namespace sdv
