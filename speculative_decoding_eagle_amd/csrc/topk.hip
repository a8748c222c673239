// A1: per-row top-k of the draft distributions (fast_topk after the per-step
// softmax, "[SGLang] Multi-Layer EAGLE" section 3).
//
// HBM-bound streaming reduction under the strict order (value desc, id asc).
// Each 256-thread block scans one slice of one row in contiguous 16 KB
// windows (16-byte non-temporal loads, four in flight per lane); every wave
// runs a threshold filter (below) over its share, and wave 0 merges the four
// per-wave lists.  Short-row batches are split over several blocks per
// row, and a one-wave kernel merges the per-slice lists.
#include <climits>
#include <cmath>

#include "common.hpp"

namespace sdv {
namespace {

constexpr int kTopkThreads = 256;

typedef float f32x4v __attribute__((ext_vector_type(4)));
// 16-byte load marked non-temporal (the probability rows are read once).
__device__ __forceinline__ float4 stream_load(const float *p) {
  const f32x4v v = __builtin_nontemporal_load(reinterpret_cast<const f32x4v *>(p));
  return make_float4(v.x, v.y, v.z, v.w);
}

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

// Per-wave candidate filter.  A wave keeps its current best K (value, id)
// sorted in LDS and a threshold = the K-th of them; elements that beat the
// threshold are appended to a per-wave LDS buffer (ballot + prefix count)
// and the buffer is folded into the best-K list whenever it fills up.  After
// the first fold the threshold is high enough that almost no element passes,
// so the scan is one compare and one ballot per 16-byte load.
constexpr int kCap = 512;                     // candidate slots per wave

template <int K>
struct WaveFilter {
  float *cv;            // [kCap] candidate values (this wave's slice of LDS)
  int *ci;              // [kCap] candidate ids
  float *tv;            // [K] best values, sorted best first
  int *ti;              // [K] best ids
  int cnt;              // candidates buffered (wave-uniform)
  float thr_v;          // K-th best value so far (wave-uniform)
  int thr_i;

  __device__ void init(float *v, int *i, float *bv, int *bi) {
    cv = v;
    ci = i;
    tv = bv;
    ti = bi;
    cnt = 0;
    thr_v = -INFINITY;
    thr_i = INT_MAX;
    if (lane_id() < K) {
      tv[lane_id()] = -INFINITY;
      ti[lane_id()] = INT_MAX;
    }
  }

  // Folds the buffered candidates into the best-K list.
  __device__ void fold() {
    __builtin_amdgcn_wave_barrier();   // candidate stores of every lane precede the reads
    SortedK<K> L;
    L.init();
    const int n = cnt + K;
    for (int x = lane_id(); x < n; x += kWave) {
      const float v = x < K ? tv[x] : cv[x - K];
      const int i = x < K ? ti[x] : ci[x - K];
      L.insert(v, i);
    }
    float keep_v = -INFINITY;
    int keep_i = INT_MAX;
    for (int r = 0; r < K; ++r) {
      float bv = L.v[0];
      int bi = L.i[0];
      wave_best(bv, bi);
      if (L.i[0] == bi && L.v[0] == bv && bi != INT_MAX) L.pop_front();
      if (lane_id() == r) {
        keep_v = bv;
        keep_i = bi;
      }
    }
    if (lane_id() < K) {
      tv[lane_id()] = keep_v;
      ti[lane_id()] = keep_i;
    }
    thr_v = __shfl(keep_v, K - 1, kWave);
    thr_i = __shfl(keep_i, K - 1, kWave);
    cnt = 0;
  }

  __device__ __forceinline__ void push(bool pred, float v, int i) {
    const unsigned long long m = __ballot(pred);
    if (m == 0ull) return;
    const int before = __popcll(m & ((1ull << lane_id()) - 1ull));
    if (pred) {
      cv[cnt + before] = v;
      ci[cnt + before] = i;
    }
    cnt += __popcll(m);
  }

  // Elements e .. e+3 (valid = false: this lane has none).
  __device__ __forceinline__ void consume4(float4 a, int e, bool valid = true) {
    const float m = fmaxf(fmaxf(a.x, a.y), fmaxf(a.z, a.w));
    // conservative pre-test: an element can only beat the threshold if m >= thr_v
    if (__ballot(valid && m >= thr_v) == 0ull) return;
    push(valid && better(a.x, e, thr_v, thr_i), a.x, e);
    push(valid && better(a.y, e + 1, thr_v, thr_i), a.y, e + 1);
    push(valid && better(a.z, e + 2, thr_v, thr_i), a.z, e + 2);
    push(valid && better(a.w, e + 3, thr_v, thr_i), a.w, e + 3);
    if (cnt > kCap - 4 * kWave) fold();
  }

  __device__ __forceinline__ void consume1(float a, int e, bool valid) {
    push(valid && better(a, e, thr_v, thr_i), a, e);
    if (cnt > kCap - kWave) fold();
  }
};

template <int K>
__global__ void __launch_bounds__(kTopkThreads)
topk_slice_kernel(const float *__restrict__ probs, int64_t rows, int V, int splits, int chunk,
                  int k, bool vec, float *__restrict__ out_v, int *__restrict__ out_i,
                  float *__restrict__ part_v, int *__restrict__ part_i) {
  constexpr int NW = kTopkThreads / kWave;
  __shared__ float s_cv[NW][kCap];
  __shared__ int s_ci[NW][kCap];
  __shared__ float s_tv[NW][K];
  __shared__ int s_ti[NW][K];
  const int64_t bid = blockIdx.x;
  const int64_t row = bid / splits;
  const int split = static_cast<int>(bid % splits);
  if (row >= rows) return;
  const float *rp = probs + row * static_cast<int64_t>(V);
  const int lo = split * chunk;
  const int hi = min(V, lo + chunk);
  const int tid = threadIdx.x;
  const int w = tid / kWave;

  WaveFilter<K> F;
  F.init(s_cv[w], s_ci[w], s_tv[w], s_ti[w]);
  if (vec) {
    // The block reads one contiguous 16 KB window per iteration: load u of
    // wave w covers 1 KB chunk 4*u + w of the window.  One stream per row
    // (rather than one per wave) and non-temporal loads (the rows are read
    // once) keep HBM efficient when a thousand rows stream at once.
    const int step = 4 * kWave;                   // floats per 1 KB chunk
    const int win = 4 * NW * step;                // floats per window
    int base = lo;
    for (; base + win <= hi; base += win) {
      const int e = base + w * step + 4 * lane_id();
      const float4 a0 = stream_load(rp + e);
      const float4 a1 = stream_load(rp + e + NW * step);
      const float4 a2 = stream_load(rp + e + 2 * NW * step);
      const float4 a3 = stream_load(rp + e + 3 * NW * step);
      F.consume4(a0, e);
      F.consume4(a1, e + NW * step);
      F.consume4(a2, e + 2 * NW * step);
      F.consume4(a3, e + 3 * NW * step);
    }
    for (int e = base + w * step + 4 * lane_id(); e - 4 * lane_id() < hi; e += NW * step) {
      const bool in = e < hi;
      const float4 a = in ? stream_load(rp + e) : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
      F.consume4(a, e, in);
    }
  } else {
    for (int e0 = lo + w * kWave; e0 < hi; e0 += NW * kWave) {
      const int e = e0 + lane_id();
      const bool in = e < hi;
      F.consume1(in ? rp[e] : -INFINITY, e, in);
    }
  }
  F.fold();
  __syncthreads();

  // wave 0 merges the four per-wave lists
  if (w == 0) {
    SortedK<K> L;
    L.init();
    for (int x = lane_id(); x < NW * K; x += kWave) L.insert(s_tv[x / K][x % K], s_ti[x / K][x % K]);
    for (int r = 0; r < K; ++r) {
      float bv = L.v[0];
      int bi = L.i[0];
      wave_best(bv, bi);
      if (L.i[0] == bi && L.v[0] == bv && bi != INT_MAX) L.pop_front();
      if (lane_id() == 0) {
        if (splits == 1) {
          if (r < k) {
            out_v[row * k + r] = bv;
            out_i[row * k + r] = bi;
          }
        } else {
          part_v[bid * K + r] = bv;
          part_i[bid * K + r] = bi;
        }
      }
    }
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
