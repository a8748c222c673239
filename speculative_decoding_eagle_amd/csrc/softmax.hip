// Processed distributions: p = softmax(logits / T) per row -- the target-side
// processing of the stochastic verify and the draft's per-step softmax
// ("[SGLang] Multi-Layer EAGLE", section 3: softmax, then fast_topk, after
// each draft pass; zero-to-sglang ch.10 section 5.1: the acceptance test
// compares the target's and the draft's probabilities of a token).
//
// HBM-bound: one workgroup of 1024 threads per row, two passes over the row.
// The first streams it once and keeps, per thread, a running maximum and the
// sum of 2^((x - max) * c) (c = log2(e) / T), moving to a larger maximum
// once per 16 entries; the 1024 partial (max, sum) pairs then merge in a
// fixed order (a butterfly across each wave, then the waves in index order),
// so the normaliser does not depend on timing.  The second pass writes
// p = 2^(x * c - m * c) * (1 / sum) with non-temporal stores.
//
// Where does the second pass read the row from?  Rows of 64 K to 132 K
// entries (V % 4 == 0) stay on chip between the passes: 24 float4 per
// thread in registers (384 KB of the CU's 512 KB register file) and the rest,
// up to 144 KB, in LDS by DMA, one workgroup per CU; each row crosses HBM
// once each way.  Other rows are read again from HBM (with a row per
// workgroup in flight on every CU the re-read misses the last-level cache:
// measured FETCH_SIZE twice the row bytes).  Both forms run the same
// arithmetic in the same order.
#include <cmath>

#include "common.hpp"

namespace sdv {
namespace {

constexpr int kSmThreads = 1024;
constexpr int kSmWaves = kSmThreads / kWave;
constexpr int kSmUnroll = 4;               // float4 loads per thread in flight in the first pass
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kStart = -1e30f;           // running maximum before any entry (finite: no inf - inf)
// On-chip rows: float4 chunk k of thread t is float4 t + k * kSmThreads of
// the row; chunks below kRegChunks live in registers, the next ones (at most
// kLdsChunks) in LDS at slot (k - kRegChunks) * kSmThreads + t.
constexpr int kRegChunks = 24;
constexpr int kLdsChunks = 9;
constexpr int kOnchipMin = 65536;                                       // entries (measured: faster from here on; below, with few rows, not)
constexpr int kOnchipMax = (kRegChunks + kLdsChunks) * kSmThreads * 4;  // 135168 entries

typedef float f32x4v __attribute__((ext_vector_type(4)));

// (m, s) absorbs (m2, s2): the pair that sums both, referred to the larger
// maximum.  Both maxima are finite (they start at kStart).
__device__ __forceinline__ void merge_ms(float &m, float &s, float m2, float s2, float c) {
  const float nm = fmaxf(m, m2);
  s = s * __builtin_amdgcn_exp2f((m - nm) * c) + s2 * __builtin_amdgcn_exp2f((m2 - nm) * c);
  m = nm;
}

// Folds entries x[0..n) into the running (m, s): one maximum move for the
// group, then one exponential per entry.
template <int NV>
__device__ __forceinline__ void absorb(const float (&x)[NV], float &m, float &s, float c) {
  float gm = x[0];
#pragma unroll
  for (int k = 1; k < NV; ++k) gm = fmaxf(gm, x[k]);
  const float nm = fmaxf(m, gm);
  const float nmc = nm * c;
  float add = 0.0f;
#pragma unroll
  for (int k = 0; k < NV; ++k) add += __builtin_amdgcn_exp2f(fmaf(x[k], c, -nmc));
  s = s * __builtin_amdgcn_exp2f((m - nm) * c) + add;
  m = nm;
}

// The (max, sum) of the row from every thread's running pair: a butterfly
// across each wave (every lane ends with the same pair), then the waves in
// index order.
__device__ __forceinline__ void row_ms(float &m, float &s, float c) {
#pragma unroll
  for (int off = kWave / 2; off >= 1; off >>= 1) {
    const float m2 = __shfl_xor(m, off, kWave);
    const float s2 = __shfl_xor(s, off, kWave);
    merge_ms(m, s, m2, s2, c);
  }
  __shared__ float s_m[kSmWaves], s_s[kSmWaves];
  const int w = threadIdx.x / kWave;
  if (lane_id() == 0) {
    s_m[w] = m;
    s_s[w] = s;
  }
  __syncthreads();
  m = s_m[0];
  s = s_s[0];
  for (int k = 1; k < kSmWaves; ++k) merge_ms(m, s, s_m[k], s_s[k], c);
}

// The on-chip form (V % 4 == 0, kOnchipMin <= V <= kOnchipMax, 16-byte
// aligned rows): one row per workgroup, nlds = the LDS chunks the row
// needs, dynamic LDS of nlds * 16 KB.  The first pass groups a thread's
// chunks as the two-pass kernel does (four float4 while its fourth one
// exists, then one at a time).  (A persistent form that loaded the next
// row's chunk into each slot as soon as its output was stored measured
// slower: the next workgroup on a CU already starts its reads while the
// last one's writes drain.)
__global__ void __launch_bounds__(kSmThreads, 1) softmax_rows_onchip_kernel(const float *__restrict__ logits, int V,
                                                                           float c, float *__restrict__ probs,
                                                                           int nlds) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int64_t row = blockIdx.x;
  const f32x4v *x4 = reinterpret_cast<const f32x4v *>(logits + row * V);
  f32x4v *p4 = reinterpret_cast<f32x4v *>(probs + row * V);
  const int tid = threadIdx.x;
  const int n4 = V / 4;
  auto has = [&](int k) __attribute__((always_inline)) { return tid + k * kSmThreads < n4; };

  // ---- the row onto the chip: the LDS chunks by DMA (inline assembly that
  // the compiler's wait placement does not see; pass 1 waits for them
  // itself; lanes past the row issue nothing), then the register chunks.
  // Register chunks past the row load the row's last float4 instead and are
  // never used: no branch, so that each one's first use waits for its own
  // load only.
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_offset(smem) + (tid / kWave) * kWave * 16);   // this wave's slot of LDS chunk 0
#pragma unroll
  for (int k2 = 0; k2 < kLdsChunks; ++k2)
    if (k2 < nlds && has(kRegChunks + k2)) dma16(x4 + tid + (kRegChunks + k2) * kSmThreads, lds0 + k2 * kSmThreads * 16);
  f32x4v v[kRegChunks];
#pragma unroll
  for (int k = 0; k < kRegChunks; ++k) v[k] = __builtin_nontemporal_load(x4 + min(tid + k * kSmThreads, n4 - 1));
  auto chunk = [&](int k) __attribute__((always_inline)) {
    if (k < kRegChunks) return v[k];
    return *reinterpret_cast<const f32x4v *>(smem + static_cast<size_t>((k - kRegChunks) * kSmThreads + tid) * 16);
  };

  // ---- pass 1
  float m = kStart, s = 0.0f;
#pragma unroll
  for (int k0 = 0; k0 < kRegChunks + kLdsChunks; k0 += kSmUnroll) {
    if (k0 == kRegChunks) asm volatile("s_waitcnt vmcnt(0)" : : : "memory");   // this wave's LDS chunks are in; LDS reads stay below
    if (has(k0 + kSmUnroll - 1)) {
      float e[4 * kSmUnroll];
#pragma unroll
      for (int u = 0; u < kSmUnroll; ++u) {
        const f32x4v x = chunk(k0 + u);
        e[4 * u + 0] = x.x;
        e[4 * u + 1] = x.y;
        e[4 * u + 2] = x.z;
        e[4 * u + 3] = x.w;
      }
      absorb(e, m, s, c);
    } else {
#pragma unroll
      for (int k = k0; k < k0 + kSmUnroll && k < kRegChunks + kLdsChunks; ++k)
        if (has(k)) {
          const f32x4v x = chunk(k);
          const float e[4] = {x.x, x.y, x.z, x.w};
          absorb(e, m, s, c);
        }
    }
  }
  row_ms(m, s, c);
  const float mc = m * c;
  const float inv = 1.0f / s;

  // ---- pass 2 from the chip
#pragma unroll
  for (int k = 0; k < kRegChunks + kLdsChunks; ++k)
    if (has(k)) {
      const f32x4v x = chunk(k);
      f32x4v o;
      o.x = __builtin_amdgcn_exp2f(fmaf(x.x, c, -mc)) * inv;
      o.y = __builtin_amdgcn_exp2f(fmaf(x.y, c, -mc)) * inv;
      o.z = __builtin_amdgcn_exp2f(fmaf(x.z, c, -mc)) * inv;
      o.w = __builtin_amdgcn_exp2f(fmaf(x.w, c, -mc)) * inv;
      __builtin_nontemporal_store(o, p4 + tid + k * kSmThreads);
    }
}

template <bool VEC>
__global__ void __launch_bounds__(kSmThreads) softmax_rows_kernel(const float *__restrict__ logits, int V, float c,
                                                                  float *__restrict__ probs) {
  const int64_t row = blockIdx.x;
  const float *x = logits + row * V;
  float *p = probs + row * V;
  const int tid = threadIdx.x;
  float m = kStart, s = 0.0f;

  // ---- pass 1: running (max, sum) of this thread's entries
  if constexpr (VEC) {
    const int n4 = V / 4;
    const f32x4v *x4 = reinterpret_cast<const f32x4v *>(x);
    int i = tid;
    for (; i + (kSmUnroll - 1) * kSmThreads < n4; i += kSmUnroll * kSmThreads) {
      f32x4v v[kSmUnroll];
#pragma unroll
      for (int u = 0; u < kSmUnroll; ++u) v[u] = x4[i + u * kSmThreads];
      float e[4 * kSmUnroll];
#pragma unroll
      for (int u = 0; u < kSmUnroll; ++u) {
        e[4 * u + 0] = v[u].x;
        e[4 * u + 1] = v[u].y;
        e[4 * u + 2] = v[u].z;
        e[4 * u + 3] = v[u].w;
      }
      absorb(e, m, s, c);
    }
    for (; i < n4; i += kSmThreads) {
      const f32x4v v = x4[i];
      const float e[4] = {v.x, v.y, v.z, v.w};
      absorb(e, m, s, c);
    }
  } else {
    for (int i = tid; i < V; i += kSmThreads) {
      const float e[1] = {x[i]};
      absorb(e, m, s, c);
    }
  }

  row_ms(m, s, c);
  const float mc = m * c;
  const float inv = 1.0f / s;

  // ---- pass 2: p = 2^(x c - m c) / sum
  if constexpr (VEC) {
    const int n4 = V / 4;
    const f32x4v *x4 = reinterpret_cast<const f32x4v *>(x);
    f32x4v *p4 = reinterpret_cast<f32x4v *>(p);
    for (int i = tid; i < n4; i += kSmThreads) {
      const f32x4v v = __builtin_nontemporal_load(x4 + i);
      f32x4v o;
      o.x = __builtin_amdgcn_exp2f(fmaf(v.x, c, -mc)) * inv;
      o.y = __builtin_amdgcn_exp2f(fmaf(v.y, c, -mc)) * inv;
      o.z = __builtin_amdgcn_exp2f(fmaf(v.z, c, -mc)) * inv;
      o.w = __builtin_amdgcn_exp2f(fmaf(v.w, c, -mc)) * inv;
      __builtin_nontemporal_store(o, p4 + i);
    }
  } else {
    for (int i = tid; i < V; i += kSmThreads) p[i] = __builtin_amdgcn_exp2f(fmaf(x[i], c, -mc)) * inv;
  }
}

}  // namespace
}  // namespace sdv

using namespace sdv;

extern "C" int32_t sdv_softmax_rows(const float *logits, int64_t rows, int32_t V, float temperature, float *probs,
                                    void *stream) {
  clear_error();
  SDV_REQUIRE(rows >= 0 && V >= 1, SDV_E_SHAPE, "softmax_rows: need rows >= 0 and V >= 1 (got %lld, %d)",
              static_cast<long long>(rows), V);
  SDV_REQUIRE(std::isfinite(temperature) && temperature > 0.0f, SDV_E_SHAPE,
              "softmax_rows: temperature must be finite and > 0 (got %g)", static_cast<double>(temperature));
  SDV_REQUIRE(rows <= 0x7FFFFFFF, SDV_E_UNSUPPORTED, "softmax_rows: at most 2^31 - 1 rows");
  if (rows == 0) return SDV_OK;
  SDV_REQUIRE(logits && probs, SDV_E_NULL, "softmax_rows: NULL pointer");
  const float c = kLog2e / temperature;
  const bool vec = V % 4 == 0 && reinterpret_cast<uintptr_t>(logits) % 16 == 0 &&
                   reinterpret_cast<uintptr_t>(probs) % 16 == 0;
  hipStream_t st = as_stream(stream);
  if (vec && V >= kOnchipMin && V <= kOnchipMax) {
    static thread_local int configured_dev = -1;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(SDV_E_HIP, "softmax_rows: no device");
    if (configured_dev != dev) {
      const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(softmax_rows_onchip_kernel),
                                               hipFuncAttributeMaxDynamicSharedMemorySize,
                                               kLdsChunks * kSmThreads * 16);
      if (e != hipSuccess) return fail(SDV_E_HIP, "softmax_rows: LDS attribute: %s", hipGetErrorString(e));
      configured_dev = dev;
    }
    const int n4 = V / 4;
    const int nlds = n4 > kRegChunks * kSmThreads ? (n4 - kRegChunks * kSmThreads + kSmThreads - 1) / kSmThreads : 0;
    hipLaunchKernelGGL(softmax_rows_onchip_kernel, dim3(static_cast<unsigned>(rows)), dim3(kSmThreads),
                       static_cast<size_t>(nlds) * kSmThreads * 16, st, logits, V, c, probs, nlds);
    return check_launch("softmax_rows_onchip_kernel");
  }
  if (vec)
    hipLaunchKernelGGL(softmax_rows_kernel<true>, dim3(static_cast<unsigned>(rows)), dim3(kSmThreads), 0, st,
                       logits, V, c, probs);
  else
    hipLaunchKernelGGL(softmax_rows_kernel<false>, dim3(static_cast<unsigned>(rows)), dim3(kSmThreads), 0, st,
                       logits, V, c, probs);
  return check_launch("softmax_rows_kernel");
}
