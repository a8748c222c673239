// A1: per-row top-k of the draft distributions (fast_topk after the per-step
// softmax, "[SGLang] Multi-Layer EAGLE" section 3).
//
// HBM-bound streaming reduction.  Each 256-thread block scans one slice of
// one row with 16-byte loads (four in flight per thread), every thread keeping
// a sorted register list of its K best (value desc, id asc); the block then
// merges those lists in K rounds of block-wide argmax.  Short-row batches are
// split over several blocks per row, and a one-wave kernel merges the
// per-slice lists.
#include <climits>
#include <cmath>

#include "common.hpp"

namespace sdv {
namespace {

constexpr int kTopkThreads = 256;

template <int K>
struct SortedK {
  float v[K];
  int i[K];

  __device__ __forceinline__ void init() {
#pragma unroll
    for (int j = 0; j < K; ++j) {
      v[j] = -INFINITY;
      i[j] = INT_MAX;
    }
  }

  // Inserts (x, xi) keeping v/i sorted best-first; no-op if not among the K best.
  __device__ __forceinline__ void insert(float x, int xi) {
    if (!better(x, xi, v[K - 1], i[K - 1])) return;
#pragma unroll
    for (int j = K - 1; j >= 1; --j) {
      const bool s = better(x, xi, v[j - 1], i[j - 1]);   // entry j-1 moves down
      const bool w = s || better(x, xi, v[j], i[j]);       // slot j is rewritten
      const float nv = s ? v[j - 1] : x;
      const int ni = s ? i[j - 1] : xi;
      v[j] = w ? nv : v[j];
      i[j] = w ? ni : i[j];
    }
    if (better(x, xi, v[0], i[0])) {
      v[0] = x;
      i[0] = xi;
    }
  }

  __device__ __forceinline__ void pop_front() {
#pragma unroll
    for (int j = 0; j < K - 1; ++j) {
      v[j] = v[j + 1];
      i[j] = i[j + 1];
    }
    v[K - 1] = -INFINITY;
    i[K - 1] = INT_MAX;
  }
};

template <int K>
__device__ __forceinline__ void consume4(SortedK<K> &L, float4 a, int e) {
  const float m = fmaxf(fmaxf(a.x, a.y), fmaxf(a.z, a.w));
  if (m >= L.v[K - 1]) {
    L.insert(a.x, e);
    L.insert(a.y, e + 1);
    L.insert(a.z, e + 2);
    L.insert(a.w, e + 3);
  }
}

// Block-wide K rounds of argmax over the threads' sorted lists; thread 0
// receives the merged list in (ov, oi).
template <int K>
__device__ void block_merge(SortedK<K> &L, float *ov, int *oi) {
  __shared__ float sv[kTopkThreads / kWave];
  __shared__ int si[kTopkThreads / kWave];
  const int w = threadIdx.x / kWave;
  const int nw = blockDim.x / kWave;
  for (int r = 0; r < K; ++r) {
    float bv = L.v[0];
    int bi = L.i[0];
    wave_best(bv, bi);
    if (lane_id() == 0) {
      sv[w] = bv;
      si[w] = bi;
    }
    __syncthreads();
    float gv = sv[0];
    int gi = si[0];
    for (int x = 1; x < nw; ++x)
      if (better(sv[x], si[x], gv, gi)) {
        gv = sv[x];
        gi = si[x];
      }
    if (L.i[0] == gi && L.v[0] == gv && gi != INT_MAX) L.pop_front();
    if (threadIdx.x == 0) {
      ov[r] = gv;
      oi[r] = gi;
    }
    __syncthreads();
  }
}

template <int K>
__global__ void __launch_bounds__(kTopkThreads)
topk_slice_kernel(const float *__restrict__ probs, int64_t rows, int V, int splits, int chunk,
                  int k, bool vec, float *__restrict__ out_v, int *__restrict__ out_i,
                  float *__restrict__ part_v, int *__restrict__ part_i) {
  const int64_t bid = blockIdx.x;
  const int64_t row = bid / splits;
  const int split = static_cast<int>(bid % splits);
  if (row >= rows) return;
  const float *rp = probs + row * static_cast<int64_t>(V);
  const int lo = split * chunk;
  const int hi = min(V, lo + chunk);

  SortedK<K> L;
  L.init();
  const int tid = threadIdx.x;
  if (vec) {
    const int step = 4 * kTopkThreads;
    int e = lo + 4 * tid;
    for (; e + 3 * step < hi; e += 4 * step) {
      const float4 a0 = *reinterpret_cast<const float4 *>(rp + e);
      const float4 a1 = *reinterpret_cast<const float4 *>(rp + e + step);
      const float4 a2 = *reinterpret_cast<const float4 *>(rp + e + 2 * step);
      const float4 a3 = *reinterpret_cast<const float4 *>(rp + e + 3 * step);
      consume4(L, a0, e);
      consume4(L, a1, e + step);
      consume4(L, a2, e + 2 * step);
      consume4(L, a3, e + 3 * step);
    }
    for (; e < hi; e += step) consume4(L, *reinterpret_cast<const float4 *>(rp + e), e);
  } else {
    for (int e = lo + tid; e < hi; e += kTopkThreads) L.insert(rp[e], e);
  }

  __shared__ float mv[K];
  __shared__ int mi[K];
  block_merge<K>(L, mv, mi);
  if (splits == 1) {
    if (tid < k) {
      out_v[row * k + tid] = mv[tid];
      out_i[row * k + tid] = mi[tid];
    }
  } else if (tid < K) {
    part_v[bid * K + tid] = mv[tid];
    part_i[bid * K + tid] = mi[tid];
  }
}

// One wave per row merges splits*K candidates.
template <int K>
__global__ void __launch_bounds__(kWave)
topk_merge_kernel(int64_t rows, int splits, int k, const float *__restrict__ part_v,
                  const int *__restrict__ part_i, float *__restrict__ out_v,
                  int *__restrict__ out_i) {
  const int64_t row = blockIdx.x;
  if (row >= rows) return;
  const int n = splits * K;
  const float *pv = part_v + row * n;
  const int *pi = part_i + row * n;
  SortedK<K> L;
  L.init();
  for (int c = lane_id(); c < n; c += kWave) L.insert(pv[c], pi[c]);
  for (int r = 0; r < k; ++r) {
    float bv = L.v[0];
    int bi = L.i[0];
    wave_best(bv, bi);
    if (L.i[0] == bi && L.v[0] == bv && bi != INT_MAX) L.pop_front();
    if (lane_id() == 0) {
      out_v[row * k + r] = bv;
      out_i[row * k + r] = bi;
    }
  }
}

struct TopkPlan {
  int K, splits, chunk;
};

TopkPlan plan_topk(int64_t rows, int V, int k) {
  TopkPlan p;
  p.K = 1;
  while (p.K < k) p.K <<= 1;
  const int64_t target = 4LL * num_cus();
  int64_t splits = rows >= target ? 1 : (target + rows - 1) / rows;
  const int64_t max_splits = V / 4096 > 0 ? V / 4096 : 1;
  if (splits > max_splits) splits = max_splits;
  int64_t chunk = (V + splits - 1) / splits;
  chunk = (chunk + 3) / 4 * 4;
  splits = (V + chunk - 1) / chunk;
  p.splits = static_cast<int>(splits);
  p.chunk = static_cast<int>(chunk);
  return p;
}

template <int K>
int32_t launch_topk(const float *probs, int64_t rows, int V, int k, const TopkPlan &p, bool vec,
                    float *out_v, int *out_i, float *part_v, int *part_i, hipStream_t st) {
  const int64_t blocks = rows * p.splits;
  hipLaunchKernelGGL(topk_slice_kernel<K>, dim3(static_cast<unsigned>(blocks)), dim3(kTopkThreads), 0,
                     st, probs, rows, V, p.splits, p.chunk, k, vec, out_v, out_i, part_v, part_i);
  int32_t rc = check_launch("topk_slice_kernel");
  if (rc != SDV_OK || p.splits == 1) return rc;
  hipLaunchKernelGGL(topk_merge_kernel<K>, dim3(static_cast<unsigned>(rows)), dim3(kWave), 0, st, rows,
                     p.splits, k, part_v, part_i, out_v, out_i);
  return check_launch("topk_merge_kernel");
}

}  // namespace
}  // namespace sdv

using namespace sdv;

extern "C" size_t sdv_draft_topk_workspace_size(int64_t rows, int32_t V, int32_t k) {
  if (rows <= 0 || V <= 0 || k <= 0 || k > 32) return 0;
  const TopkPlan p = plan_topk(rows, V, k);
  if (p.splits == 1) return 0;
  Carver c(nullptr);
  c.take<float>(static_cast<size_t>(rows) * p.splits * p.K);
  c.take<int>(static_cast<size_t>(rows) * p.splits * p.K);
  return c.bytes();
}

extern "C" int32_t sdv_draft_topk(const float *probs, int64_t rows, int32_t V, int32_t k,
                                  float *topk_p, int32_t *topk_id, void *ws, size_t ws_bytes,
                                  void *stream) {
  clear_error();
  SDV_REQUIRE(rows >= 0 && V >= 1 && k >= 1 && k <= V, SDV_E_SHAPE,
              "draft_topk: need rows >= 0 and 1 <= k <= V (rows=%lld V=%d k=%d)",
              static_cast<long long>(rows), V, k);
  SDV_REQUIRE(k <= 32, SDV_E_UNSUPPORTED, "draft_topk: k=%d above 32", k);
  SDV_REQUIRE(V < INT_MAX - 4096, SDV_E_UNSUPPORTED, "draft_topk: V too large");
  SDV_REQUIRE(rows <= (1LL << 30), SDV_E_UNSUPPORTED, "draft_topk: too many rows");
  if (rows == 0) return SDV_OK;
  SDV_REQUIRE(probs && topk_p && topk_id, SDV_E_NULL, "draft_topk: NULL pointer");
  const TopkPlan p = plan_topk(rows, V, k);
  const size_t need = sdv_draft_topk_workspace_size(rows, V, k);
  SDV_REQUIRE(ws_bytes >= need && (need == 0 || ws), SDV_E_WORKSPACE,
              "draft_topk: workspace of %zu bytes needed", need);
  Carver c(ws);
  float *part_v = c.take<float>(static_cast<size_t>(rows) * p.splits * p.K);
  int *part_i = c.take<int>(static_cast<size_t>(rows) * p.splits * p.K);
  const bool vec = (V % 4 == 0) && (reinterpret_cast<uintptr_t>(probs) % 16 == 0);
  hipStream_t st = as_stream(stream);
  switch (p.K) {
    case 1: return launch_topk<1>(probs, rows, V, k, p, vec, topk_p, topk_id, part_v, part_i, st);
    case 2: return launch_topk<2>(probs, rows, V, k, p, vec, topk_p, topk_id, part_v, part_i, st);
    case 4: return launch_topk<4>(probs, rows, V, k, p, vec, topk_p, topk_id, part_v, part_i, st);
    case 8: return launch_topk<8>(probs, rows, V, k, p, vec, topk_p, topk_id, part_v, part_i, st);
    case 16: return launch_topk<16>(probs, rows, V, k, p, vec, topk_p, topk_id, part_v, part_i, st);
    default: return launch_topk<32>(probs, rows, V, k, p, vec, topk_p, topk_id, part_v, part_i, st);
  }
}
