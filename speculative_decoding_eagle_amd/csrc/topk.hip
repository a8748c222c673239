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
constexpr int kLoads = 4;        // 16-byte loads per lane in flight per window

typedef float f32x4v __attribute__((ext_vector_type(4)));

// The wave sort below replaces K rounds of wave-wide best-of selection
// (six exchange steps each) from this K on, where it is the cheaper of the
// two.
constexpr int kSortNetK = 8;

// Sorts one (value, id) pair per lane across the wave under the strict
// order, best first: lane 0 ends with the best pair.  A bitonic network of
// 21 compare-exchange stages between lanes l and l ^ stride; equal pairs
// (only the (-inf, INT_MAX) padding can be equal) never swap.
__device__ __forceinline__ void wave_sort_best_first(float &v, int &i) {
  const int lane = lane_id();
#pragma unroll
  for (int size = 2; size <= kWave; size <<= 1) {
#pragma unroll
    for (int stride = size / 2; stride > 0; stride >>= 1) {
      const float ov = __shfl_xor(v, stride, kWave);
      const int oi = __shfl_xor(i, stride, kWave);
      const bool best_first = (lane & size) == 0;            // this block's direction
      const bool lower = (lane & stride) == 0;                // this lane's place in the pair
      const bool take = (lower == best_first) ? better(ov, oi, v, i) : better(v, i, ov, oi);
      v = take ? ov : v;
      i = take ? oi : i;
    }
  }
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
template <int K, int CAP>
struct WaveFilter {
  float *cv;            // [CAP] candidate values (this wave's slice of LDS)
  int *ci;              // [CAP] candidate ids
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
  __device__ __forceinline__ void fold() {
    __builtin_amdgcn_wave_barrier();   // candidate stores of every lane precede the reads
    if (K >= kSortNetK && cnt + K <= kWave) {
      // one candidate (or list entry) per lane: a wave sort gives the new list
      const int x = lane_id();
      float v = -INFINITY;
      int i = INT_MAX;
      if (x < K) {
        v = tv[x];
        i = ti[x];
      } else if (x < K + cnt) {
        v = cv[x - K];
        i = ci[x - K];
      }
      wave_sort_best_first(v, i);
      if (x < K) {
        tv[x] = v;
        ti[x] = i;
      }
      thr_v = __shfl(v, K - 1, kWave);
      thr_i = __shfl(i, K - 1, kWave);
      cnt = 0;
      return;
    }
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

  // Raises the threshold, before anything is buffered, to the K-th largest
  // of the lanes' maxima over a first stretch of the wave's elements.  K of
  // the wave's elements reach that value, so each of its K best does too;
  // with the id bound at INT_MAX, elements equal to it still pass.  This
  // spares the folds that a threshold at -inf would take on the first
  // elements.
  __device__ void seed(float lane_max) {
    float v = lane_max, kth = -INFINITY;
    for (int r = 0; r < K; ++r) {
      float m = v;
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) m = vmax(m, __shfl_xor(m, off, kWave));
      const unsigned long long hit = __ballot(v == m);
      if (lane_id() == __ffsll(static_cast<long long>(hit)) - 1) v = -INFINITY;
      kth = m;
    }
    thr_v = kth;
    thr_i = INT_MAX;
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

  // n elements per lane at ids e .. e+n-1 (valid = false: this lane has
  // none); mx is the largest of them.  Nothing happens unless some lane's
  // mx reaches the threshold.  With EACH, a ballot on x >= thr_v (one
  // compare) skips the exact test of element j wherever no lane reaches the
  // threshold (cheaper when n is large); then the buffer is folded if
  // another n elements per lane might not fit.
  template <int n, bool EACH>
  __device__ __forceinline__ void offer(const float *xs, float mx, int e, bool valid) {
    if (__ballot(valid && mx >= thr_v) == 0ull) return;
#pragma unroll
    for (int j = 0; j < n; ++j) {
      if (!EACH || __ballot(valid && xs[j] >= thr_v) != 0ull)
        push(valid && better(xs[j], e + j, thr_v, thr_i), xs[j], e + j);
    }
    if (cnt > CAP - n * kWave) fold();
  }
};

// What a row holds: probabilities (fp32), or logits (fp32 or bf16) that the
// kernel turns into softmax(logits / T) of the selected entries.
enum : int { kInProbs = 0, kInLogitsF32 = 1, kInLogitsBf16 = 2 };

// Running softmax normaliser in log2 units: m = largest logit seen, s = sum
// of 2^((x - m) * c) with c = log2(e) / T.  Entries at -inf add nothing;
// m = -inf while nothing finite has been seen (then s = 0).
struct Norm {
  float m = -INFINITY, s = 0.f;

  // Adds the n entries of xs, whose largest is mx.  Branch-free: the old sum
  // is rescaled by 2^((m - m') c) (0 while m = -inf), each term is
  // 2^(x c - m' c) in one fma and one exp.
  template <int n>
  __device__ __forceinline__ void add(const float (&xs)[n], float mx, float c) {
    const float mn = vmax(m, mx);
    const float mc = mn == -INFINITY ? 0.f : mn * c;
    float t0 = __builtin_amdgcn_exp2f(fmaf(xs[0], c, -mc)), t1 = 0.f;
    if constexpr (n > 1) t1 = __builtin_amdgcn_exp2f(fmaf(xs[1], c, -mc));
#pragma unroll
    for (int j = 2; j < n; j += 2) {
      t0 += __builtin_amdgcn_exp2f(fmaf(xs[j], c, -mc));
      if (j + 1 < n) t1 += __builtin_amdgcn_exp2f(fmaf(xs[j + 1], c, -mc));
    }
    s = fmaf(s, __builtin_amdgcn_exp2f(fmaf(m, c, -mc)), t0 + t1);
    m = mn;
  }
  // this <- this (+) o, this one's terms first
  __device__ __forceinline__ void merge(float om, float os, float c) {
    const float M = vmax(m, om);
    if (M == -INFINITY) return;
    const float a = m == -INFINITY ? 0.f : s * __builtin_amdgcn_exp2f((m - M) * c);
    const float b = om == -INFINITY ? 0.f : os * __builtin_amdgcn_exp2f((om - M) * c);
    m = M;
    s = a + b;
  }
};

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// One slice [lo, hi) of one row.  IN: what the row holds (above).
template <int K, int IN>
__global__ void __launch_bounds__(kTopkThreads)
topk_slice_kernel(const void *__restrict__ rows_in, int64_t rows, int V, int splits, int chunk,
                  int k, bool vec, float c2, float *__restrict__ out_v, int *__restrict__ out_i,
                  float *__restrict__ part_v, int *__restrict__ part_i, float2 *__restrict__ part_n) {
  constexpr int NW = kTopkThreads / kWave;
  constexpr bool LOGITS = IN != kInProbs;
  constexpr int EPL = IN == kInLogitsBf16 ? 8 : 4;          // elements per 16-byte load
  // Software pipelined windows (the next window's loads issued before this
  // one is processed), filtered element by element (see offer) with a
  // larger candidate buffer: for bf16 rows, which carry twice the elements
  // per byte, and for K <= 4, where the second set of load registers still
  // leaves six workgroups per CU.  Otherwise one window at a time.
  constexpr bool PIPE = EPL == 8 || K <= 4;
  constexpr int CAP = PIPE ? 768 : 512;                     // candidate slots per wave
  __shared__ float s_cv[NW][CAP];
  __shared__ int s_ci[NW][CAP];
  __shared__ float s_tv[NW][K];
  __shared__ int s_ti[NW][K];
  __shared__ float2 s_norm[NW];
  const int64_t bid = blockIdx.x;
  const int64_t row = bid / splits;
  const int split = static_cast<int>(bid % splits);
  if (row >= rows) return;
  const int lo = split * chunk;
  const int hi = min(V, lo + chunk);
  const int tid = threadIdx.x;
  const int w = tid / kWave;
  const float *rp32 = static_cast<const float *>(rows_in) + row * static_cast<int64_t>(V);
  const uint16_t *rp16 = static_cast<const uint16_t *>(rows_in) + row * static_cast<int64_t>(V);

  WaveFilter<K, CAP> F;
  F.init(s_cv[w], s_ci[w], s_tv[w], s_ti[w]);
  Norm nm;
  // one 16-byte load: EPL elements starting at element e
  auto load = [&](int e) {
    return IN == kInLogitsBf16 ? __builtin_nontemporal_load(reinterpret_cast<const f32x4v *>(rp16 + e))
                               : __builtin_nontemporal_load(reinterpret_cast<const f32x4v *>(rp32 + e));
  };
  auto unpack = [&](const f32x4v &u, float *x) {
    if constexpr (IN == kInLogitsBf16) {
      const uint32_t wd[4] = {__float_as_uint(u.x), __float_as_uint(u.y), __float_as_uint(u.z),
                              __float_as_uint(u.w)};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x[2 * j] = bf16_to_f32(wd[j] & 0xffffu);
        x[2 * j + 1] = __uint_as_float(wd[j] & 0xffff0000u);
      }
    } else {
      x[0] = u.x;
      x[1] = u.y;
      x[2] = u.z;
      x[3] = u.w;
    }
  };
  if (vec) {
    // The block reads one contiguous window of kLoads * 4 KB per iteration:
    // load u of wave w covers 1 KB chunk 4*u + w of the window.  One stream per row
    // (rather than one per wave) and non-temporal loads (the rows are read
    // once) keep HBM efficient when a thousand rows stream at once.  The
    // loads are all in flight before the first is used, one ballot
    // tests the lane maxima of the window against the threshold, and the
    // normaliser takes the window in one update.
    constexpr int step = EPL * kWave;             // elements per 1 KB chunk
    constexpr int win = kLoads * NW * step;       // elements per window
    // the window at base, its loads in r
    auto window = [&](int base, const f32x4v (&r)[kLoads]) {
      const int e = base + w * step + EPL * lane_id();
      float x[kLoads * EPL];
#pragma unroll
      for (int u = 0; u < kLoads; ++u) unpack(r[u], x + u * EPL);
      float lmx[kLoads];
#pragma unroll
      for (int u = 0; u < kLoads; ++u) {
        lmx[u] = x[u * EPL];
#pragma unroll
        for (int j = 1; j < EPL; ++j) lmx[u] = vmax(lmx[u], x[u * EPL + j]);
      }
      float mx = lmx[0];
#pragma unroll
      for (int u = 1; u < kLoads; ++u) mx = vmax(mx, lmx[u]);
      if (base == lo) F.seed(mx);                 // the first window's lane maxima
      if (__ballot(mx >= F.thr_v) != 0ull) {
#pragma unroll
        for (int u = 0; u < kLoads; ++u) F.template offer<EPL, PIPE>(x + u * EPL, lmx[u], e + u * NW * step, true);
      }
      if constexpr (LOGITS) nm.add(x, mx, c2);
    };
    auto issue = [&](int base, f32x4v (&r)[kLoads]) {
      const int e = base + w * step + EPL * lane_id();
#pragma unroll
      for (int u = 0; u < kLoads; ++u) r[u] = load(e + u * NW * step);
    };
    int base = lo;
    if constexpr (PIPE) {
      if (base + win <= hi) {
        // the next window's loads are in flight while this one is processed
        f32x4v cur[kLoads], nxt[kLoads];
        issue(base, cur);
        for (; base + 2 * win <= hi; base += win) {
          issue(base + win, nxt);
          __builtin_amdgcn_sched_barrier(0);
          window(base, cur);
#pragma unroll
          for (int u = 0; u < kLoads; ++u) cur[u] = nxt[u];
        }
        window(base, cur);
        base += win;
      }
    } else {
      for (; base + win <= hi; base += win) {
        f32x4v cur[kLoads];
        issue(base, cur);
        __builtin_amdgcn_sched_barrier(0);
        window(base, cur);
      }
    }
    for (int e = base + w * step + EPL * lane_id(); e - EPL * lane_id() < hi; e += NW * step) {
      const bool in = e < hi;
      float x[EPL];
      if (in) {
        unpack(load(e), x);
      } else {
#pragma unroll
        for (int j = 0; j < EPL; ++j) x[j] = -INFINITY;
      }
      float mx = x[0];
#pragma unroll
      for (int j = 1; j < EPL; ++j) mx = vmax(mx, x[j]);
      F.template offer<EPL, PIPE>(x, mx, e, in);
      if constexpr (LOGITS) {
        if (in) nm.add(x, mx, c2);
      }
    }
  } else {
    for (int e0 = lo + w * kWave; e0 < hi; e0 += NW * kWave) {
      const int e = e0 + lane_id();
      const bool in = e < hi;
      float x[1] = {-INFINITY};
      if (in) x[0] = IN == kInLogitsBf16 ? bf16_to_f32(rp16[e]) : rp32[e];
      F.template offer<1, false>(x, x[0], e, in);
      if constexpr (LOGITS) {
        if (in) nm.add(x, x[0], c2);
      }
    }
  }
  F.fold();
  if constexpr (LOGITS) {
    // the wave's lanes in butterfly order, then the waves in order
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const float om = __shfl_xor(nm.m, off, kWave), os = __shfl_xor(nm.s, off, kWave);
      if (lane_id() & off) {
        Norm t;
        t.m = om;
        t.s = os;
        t.merge(nm.m, nm.s, c2);
        nm = t;
      } else {
        nm.merge(om, os, c2);
      }
    }
    if (lane_id() == 0) s_norm[w] = make_float2(nm.m, nm.s);
  }
  __syncthreads();

  // wave 0 merges the four per-wave lists
  if (w == 0) {
    Norm tot;
    if constexpr (LOGITS) {
#pragma unroll
      for (int x = 0; x < NW; ++x) tot.merge(s_norm[x].x, s_norm[x].y, c2);
    }
    auto emit = [&](int r, float bv, int bi) {
      if (splits == 1) {
        if (r < k) {
          out_v[row * k + r] = LOGITS ? __builtin_amdgcn_exp2f((bv - tot.m) * c2) / tot.s : bv;
          out_i[row * k + r] = bi;
        }
      } else {
        part_v[bid * K + r] = bv;
        part_i[bid * K + r] = bi;
      }
    };
    if constexpr (K >= kSortNetK && NW * K <= kWave) {
      // the four lists fit one per lane: one wave sort, lanes 0 .. K-1 emit
      const int x = lane_id();
      float bv = x < NW * K ? s_tv[x / K][x % K] : -INFINITY;
      int bi = x < NW * K ? s_ti[x / K][x % K] : INT_MAX;
      wave_sort_best_first(bv, bi);
      if (x < K) emit(x, bv, bi);
    } else {
      SortedK<K> L;
      L.init();
      for (int x = lane_id(); x < NW * K; x += kWave) L.insert(s_tv[x / K][x % K], s_ti[x / K][x % K]);
      for (int r = 0; r < K; ++r) {
        float bv = L.v[0];
        int bi = L.i[0];
        wave_best(bv, bi);
        if (L.i[0] == bi && L.v[0] == bv && bi != INT_MAX) L.pop_front();
        if (lane_id() == 0) emit(r, bv, bi);
      }
    }
    if (LOGITS && splits > 1 && lane_id() == 0) part_n[bid] = make_float2(tot.m, tot.s);
  }
}

// One wave per row merges splits*K candidates (and, for logits, the splits'
// normalisers in split order).
template <int K, bool LOGITS>
__global__ void __launch_bounds__(kWave)
topk_merge_kernel(int64_t rows, int splits, int k, float c2, const float *__restrict__ part_v,
                  const int *__restrict__ part_i, const float2 *__restrict__ part_n, float *__restrict__ out_v,
                  int *__restrict__ out_i) {
  const int64_t row = blockIdx.x;
  if (row >= rows) return;
  const int n = splits * K;
  const float *pv = part_v + row * n;
  const int *pi = part_i + row * n;
  Norm tot;
  if constexpr (LOGITS) {
    for (int x = 0; x < splits; ++x) {
      const float2 t = part_n[row * splits + x];
      tot.merge(t.x, t.y, c2);
    }
  }
  auto emit = [&](int r, float bv, int bi) {
    out_v[row * k + r] = LOGITS ? __builtin_amdgcn_exp2f((bv - tot.m) * c2) / tot.s : bv;
    out_i[row * k + r] = bi;
  };
  if (K >= kSortNetK && n <= kWave) {
    const int x = lane_id();
    float bv = x < n ? pv[x] : -INFINITY;
    int bi = x < n ? pi[x] : INT_MAX;
    wave_sort_best_first(bv, bi);
    if (x < k) emit(x, bv, bi);
    return;
  }
  SortedK<K> L;
  L.init();
  for (int c = lane_id(); c < n; c += kWave) L.insert(pv[c], pi[c]);
  for (int r = 0; r < k; ++r) {
    float bv = L.v[0];
    int bi = L.i[0];
    wave_best(bv, bi);
    if (L.i[0] == bi && L.v[0] == bv && bi != INT_MAX) L.pop_front();
    if (lane_id() == 0) emit(r, bv, bi);
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
  chunk = (chunk + 7) / 8 * 8;                       // whole 16-byte loads of fp32 and bf16
  splits = (V + chunk - 1) / chunk;
  p.splits = static_cast<int>(splits);
  p.chunk = static_cast<int>(chunk);
  return p;
}

size_t topk_workspace(int64_t rows, int V, int k, bool logits) {
  const TopkPlan p = plan_topk(rows, V, k);
  if (p.splits == 1) return 0;
  Carver c(nullptr);
  c.take<float>(static_cast<size_t>(rows) * p.splits * p.K);
  c.take<int>(static_cast<size_t>(rows) * p.splits * p.K);
  if (logits) c.take<float2>(static_cast<size_t>(rows) * p.splits);
  return c.bytes();
}

template <int K, int IN>
int32_t launch_topk(const void *rows_in, int64_t rows, int V, int k, const TopkPlan &p, bool vec, float c2,
                    float *out_v, int *out_i, float *part_v, int *part_i, float2 *part_n, hipStream_t st) {
  const int64_t blocks = rows * p.splits;
  hipLaunchKernelGGL((topk_slice_kernel<K, IN>), dim3(static_cast<unsigned>(blocks)), dim3(kTopkThreads), 0,
                     st, rows_in, rows, V, p.splits, p.chunk, k, vec, c2, out_v, out_i, part_v, part_i, part_n);
  int32_t rc = check_launch("topk_slice_kernel");
  if (rc != SDV_OK || p.splits == 1) return rc;
  hipLaunchKernelGGL((topk_merge_kernel<K, IN != kInProbs>), dim3(static_cast<unsigned>(rows)), dim3(kWave), 0,
                     st, rows, p.splits, k, c2, part_v, part_i, part_n, out_v, out_i);
  return check_launch("topk_merge_kernel");
}

// Common checks and dispatch of both entry points.
int32_t run_topk(const char *what, int IN, const void *rows_in, int64_t rows, int32_t V, int32_t k, float c2,
                 float *topk_p, int32_t *topk_id, void *ws, size_t ws_bytes, void *stream) {
  SDV_REQUIRE(rows >= 0 && V >= 1 && k >= 1 && k <= V, SDV_E_SHAPE,
              "%s: need rows >= 0 and 1 <= k <= V (rows=%lld V=%d k=%d)", what, static_cast<long long>(rows), V,
              k);
  SDV_REQUIRE(k <= 32, SDV_E_UNSUPPORTED, "%s: k=%d above 32", what, k);
  SDV_REQUIRE(V < INT_MAX - 4096, SDV_E_UNSUPPORTED, "%s: V too large", what);
  SDV_REQUIRE(rows <= (1LL << 30), SDV_E_UNSUPPORTED, "%s: too many rows", what);
  if (rows == 0) return SDV_OK;
  SDV_REQUIRE(rows_in && topk_p && topk_id, SDV_E_NULL, "%s: NULL pointer", what);
  const TopkPlan p = plan_topk(rows, V, k);
  const size_t need = topk_workspace(rows, V, k, IN != kInProbs);
  SDV_REQUIRE(ws_bytes >= need && (need == 0 || ws), SDV_E_WORKSPACE, "%s: workspace of %zu bytes needed", what,
              need);
  Carver c(ws);
  float *part_v = c.take<float>(static_cast<size_t>(rows) * p.splits * p.K);
  int *part_i = c.take<int>(static_cast<size_t>(rows) * p.splits * p.K);
  float2 *part_n = IN != kInProbs ? c.take<float2>(static_cast<size_t>(rows) * p.splits) : nullptr;
  const int epl = IN == kInLogitsBf16 ? 8 : 4;
  const bool vec = (V % epl == 0) && (reinterpret_cast<uintptr_t>(rows_in) % 16 == 0);
  hipStream_t st = as_stream(stream);
#define SDV_TOPK_IN(KK)                                                                                          \
  (IN == kInProbs        ? launch_topk<KK, kInProbs>(rows_in, rows, V, k, p, vec, c2, topk_p, topk_id, part_v,     \
                                                     part_i, part_n, st)                                         \
   : IN == kInLogitsF32 ? launch_topk<KK, kInLogitsF32>(rows_in, rows, V, k, p, vec, c2, topk_p, topk_id, part_v, \
                                                         part_i, part_n, st)                                     \
                         : launch_topk<KK, kInLogitsBf16>(rows_in, rows, V, k, p, vec, c2, topk_p, topk_id,       \
                                                          part_v, part_i, part_n, st))
  switch (p.K) {
    case 1: return SDV_TOPK_IN(1);
    case 2: return SDV_TOPK_IN(2);
    case 4: return SDV_TOPK_IN(4);
    case 8: return SDV_TOPK_IN(8);
    case 16: return SDV_TOPK_IN(16);
    default: return SDV_TOPK_IN(32);
  }
#undef SDV_TOPK_IN
}

}  // namespace
}  // namespace sdv

using namespace sdv;

extern "C" size_t sdv_draft_topk_workspace_size(int64_t rows, int32_t V, int32_t k) {
  if (rows <= 0 || V <= 0 || k <= 0 || k > 32) return 0;
  return topk_workspace(rows, V, k, false);
}

extern "C" int32_t sdv_draft_topk(const float *probs, int64_t rows, int32_t V, int32_t k,
                                  float *topk_p, int32_t *topk_id, void *ws, size_t ws_bytes,
                                  void *stream) {
  clear_error();
  return run_topk("draft_topk", kInProbs, probs, rows, V, k, 0.f, topk_p, topk_id, ws, ws_bytes, stream);
}

extern "C" size_t sdv_draft_topk_logits_workspace_size(int64_t rows, int32_t V, int32_t k) {
  if (rows <= 0 || V <= 0 || k <= 0 || k > 32) return 0;
  return topk_workspace(rows, V, k, true);
}

extern "C" int32_t sdv_draft_topk_logits(const void *logits, int32_t dtype, int64_t rows, int32_t V, int32_t k,
                                         float temperature, float *topk_p, int32_t *topk_id, void *ws,
                                         size_t ws_bytes, void *stream) {
  clear_error();
  SDV_REQUIRE(dtype == SDV_DTYPE_F32 || dtype == SDV_DTYPE_BF16, SDV_E_UNSUPPORTED,
              "draft_topk_logits: dtype %d not fp32 or bf16", dtype);
  SDV_REQUIRE(temperature > 0.f && std::isfinite(temperature), SDV_E_SHAPE,
              "draft_topk_logits: temperature must be positive");
  const float c2 = 1.4426950408889634f / temperature;
  return run_topk("draft_topk_logits", dtype == SDV_DTYPE_BF16 ? kInLogitsBf16 : kInLogitsF32, logits, rows, V,
                  k, c2, topk_p, topk_id, ws, ws_bytes, stream);
}
