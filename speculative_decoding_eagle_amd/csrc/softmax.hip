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
// so the normaliser does not depend on timing.  The second pass reads the
// row again and writes p = 2^(x * c - m * c) * (1 / sum) with non-temporal
// stores.  The second read comes from HBM too (measured: FETCH_SIZE twice
// the row bytes, also with one workgroup per CU, whose rows in flight would
// fit the last-level cache): the kernel moves 1.5x the algorithmic bytes.
#include <cmath>

#include "common.hpp"

namespace sdv {
namespace {

constexpr int kSmThreads = 1024;
constexpr int kSmWaves = kSmThreads / kWave;
constexpr int kSmUnroll = 4;               // float4 loads per thread in flight in the first pass
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kStart = -1e30f;           // running maximum before any entry (finite: no inf - inf)

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

  // ---- the row's (max, sum): butterfly within each wave (every lane ends
  // with the same pair), then the waves in index order
#pragma unroll
  for (int off = kWave / 2; off >= 1; off >>= 1) {
    const float m2 = __shfl_xor(m, off, kWave);
    const float s2 = __shfl_xor(s, off, kWave);
    merge_ms(m, s, m2, s2, c);
  }
  __shared__ float s_m[kSmWaves], s_s[kSmWaves];
  const int w = tid / kWave;
  if (lane_id() == 0) {
    s_m[w] = m;
    s_s[w] = s;
  }
  __syncthreads();
  m = s_m[0];
  s = s_s[0];
  for (int k = 1; k < kSmWaves; ++k) merge_ms(m, s, s_m[k], s_s[k], c);
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
  if (vec)
    hipLaunchKernelGGL(softmax_rows_kernel<true>, dim3(static_cast<unsigned>(rows)), dim3(kSmThreads), 0, st,
                       logits, V, c, probs);
  else
    hipLaunchKernelGGL(softmax_rows_kernel<false>, dim3(static_cast<unsigned>(rows)), dim3(kSmThreads), 0, st,
                       logits, V, c, probs);
  return check_launch("softmax_rows_kernel");
}
