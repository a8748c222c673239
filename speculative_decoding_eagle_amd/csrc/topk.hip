// A1: per-row top-k of the draft distributions (fast_topk after the per-step
// softmax, "[SGLang] Multi-Layer EAGLE" section 3).
//
// HBM-bound streaming reduction under the strict order (value desc, id asc).
// Each 256-thread block scans its segments in contiguous 8 KB windows
// (16-byte non-temporal loads, two per lane, the next window's in flight
// while this one is processed); every wave runs a threshold filter (below)
// over its share, and wave 0 merges the four per-wave lists.  With many rows
// per CU a block scans one row; otherwise every block scans the same number
// of elements of the rows laid end to end, and the last segment of a row to
// finish merges the row's lists (no second launch).
#include <climits>
#include <cmath>

#include "common.hpp"

namespace sdv {
namespace {

constexpr int kTopkThreads = 256;
// 16-byte loads per lane in flight per window.  HBM serves a full chip of
// streams fastest with about 6-8 MB in flight: with five blocks per CU, two
// loads per lane per window (four with the next window's) measured 92 us
// against 95-97 with four and 102-103 with one for 1056 rows of 128256 fp32
// probabilities, 94 against 109 for fp32 logits and 62-66 against 69-71 for
// bf16 logits (a plain grid-stride read of the same bytes: 6.9 TB/s with
// two loads per lane, 5.8 with four, 5.2 with eight).
constexpr int kLoads = 2;

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
template <int K, int CAP, int FOLD_AT>
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
    if (cnt >= FOLD_AT || cnt > CAP - n * kWave) fold();
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

// Candidates buffered before a fold: low enough that the threshold keeps up
// with the running K-th best (a threshold left at its seed lets hundreds of
// elements per wave through), and for K >= kSortNetK low enough that the
// fold is one wave sort.
template <int K>
constexpr int fold_at() {
  return K >= kSortNetK ? (kWave - 2 * K > 16 ? kWave - 2 * K : 16) : 48;
}

// Counters at the start of the workspace, one per cut row (fewer than the
// CUs), for any shape: what one call leaves there (zeros) is what the next
// expects.
constexpr int64_t kTopkRowsMax = 16384;
constexpr unsigned kTopkSpin = 1u << 20;   // polls of a published word before giving up

// A published entry is one 64-bit word, written and read with single
// relaxed atomics at device scope: the value's bits, then id + 1, so that
// no entry is zero and zero means "not yet visible".  (A normaliser (m, s)
// is never zero either: s >= 1 whenever m is finite.)  The flag is the
// value itself, so no fence is needed: a device-scope release or acquire
// would write back or invalidate a whole L2 per segment.
__device__ __forceinline__ unsigned long long pack_entry(float v, int i) {
  return (static_cast<unsigned long long>(__float_as_uint(v)) << 32) | (static_cast<unsigned>(i) + 1u);
}
__device__ __forceinline__ unsigned long long pack_norm(float m, float s) {
  return (static_cast<unsigned long long>(__float_as_uint(m)) << 32) | __float_as_uint(s);
}
__device__ __forceinline__ void put_word(unsigned long long *p, unsigned long long w) {
  __hip_atomic_store(p, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// The word at p once its writer's store is visible (at most `limit` polls;
// late is set if it never became so, and the word then reads as 0).
__device__ __forceinline__ unsigned long long await_word(unsigned long long *p, unsigned limit, bool &late) {
  for (unsigned spins = 0; spins < limit; ++spins) {
    const unsigned long long w = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (w != 0ull) return w;
    __builtin_amdgcn_s_sleep(1);
  }
  late = true;
  return 0ull;
}

// The K best of n (value, id) pairs, best first, into lanes 0 .. K-1 (other
// lanes: padding).  get(c, v, i) yields pair c.  One wave.
template <int K, typename Get>
__device__ __forceinline__ void wave_best_k(int n, Get &&get, float &bv, int &bi) {
  const int x = lane_id();
  if (K >= kSortNetK && n <= kWave) {
    bv = -INFINITY;
    bi = INT_MAX;
    if (x < n) get(x, bv, bi);
    wave_sort_best_first(bv, bi);
    return;
  }
  SortedK<K> L;
  L.init();
  for (int c = x; c < n; c += kWave) {
    float v;
    int i;
    get(c, v, i);
    L.insert(v, i);
  }
  bv = -INFINITY;
  bi = INT_MAX;
  for (int r = 0; r < K; ++r) {
    float v = L.v[0];
    int i = L.i[0];
    wave_best(v, i);
    if (L.i[0] == i && L.v[0] == v && i != INT_MAX) L.pop_front();
    if (x == r) {
      bv = v;
      bi = i;
    }
  }
}

// Block j < nwhole scans row j whole.  The rows after those (fewer than
// one per CU) are laid end to end and cut into pieces of per < V elements:
// block nwhole + j scans piece j, part of one row or the tail of one row
// and the head of the next, so that with rows = q * CUs + r each CU gets q
// whole rows and an equal share of the r others.  A whole-row segment
// writes its result.  A row cut into several segments (at most maxseg) has
// each segment publish its K best (and, for logits, its normaliser) to the
// workspace as flagged words and count itself on the row's counter; the
// segment that counts last merges the lists as their words land (the K
// best under the strict order do not depend on the merge order;
// normalisers are merged in segment order) and sets the words and the
// counter back to zero.  A wait that gives up (after wait_limit polls)
// writes NaN / -1 for the row and sets SDV_STATUS_TOPK_MERGE_WAIT in the
// workspace header.  IN: what the rows hold (above).
template <int K, int IN>
__global__ void __launch_bounds__(kTopkThreads)
topk_kernel(const void *__restrict__ rows_in, int64_t rows, int V, int64_t nwhole, int64_t per, int maxseg, int k,
            bool vec,
            float c2, float *__restrict__ out_v, int *__restrict__ out_i, unsigned *__restrict__ cnt,
            unsigned long long *__restrict__ part, unsigned long long *__restrict__ part_n,
            unsigned *__restrict__ status, unsigned wait_limit) {
  constexpr int NW = kTopkThreads / kWave;
  constexpr bool LOGITS = IN != kInProbs;
  constexpr int EPL = IN == kInLogitsBf16 ? 8 : 4;          // elements per 16-byte load
  // Software pipelined windows (the next window's loads are issued before
  // this one is processed), filtered element by element (see offer) with a
  // larger candidate buffer, up to K = 8 (bf16: 16); larger K keep one
  // window at a time, whose registers the K-lists need.
  constexpr bool PIPE = K <= 8 || (EPL == 8 && K <= 16);
  constexpr int CAP = PIPE ? 768 : 512;                     // candidate slots per wave
  __shared__ float s_cv[NW][CAP];
  __shared__ int s_ci[NW][CAP];
  __shared__ float s_tv[NW][K];
  __shared__ int s_ti[NW][K];
  __shared__ float2 s_norm[NW];
  const int64_t bid = blockIdx.x;
  const int tid = threadIdx.x;
  const int w = tid / kWave;
  const int x = lane_id();

  // Segment [lo, hi) of one row.  Called at most twice per block (per < V),
  // without a loop: a loop back edge keeps hoisted per-lane values live
  // across the window loop and costs a workgroup per CU.
  auto segment = [&](const int64_t row, const int lo, const int hi) __attribute__((always_inline)) {
    const float *rp32 = static_cast<const float *>(rows_in) + row * static_cast<int64_t>(V);
    const uint16_t *rp16 = static_cast<const uint16_t *>(rows_in) + row * static_cast<int64_t>(V);

    WaveFilter<K, CAP, fold_at<K>()> F;
    F.init(s_cv[w], s_ci[w], s_tv[w], s_ti[w]);
    Norm nm;
    // one 16-byte load: EPL elements starting at element e
    auto load = [&](int e) {
      return IN == kInLogitsBf16 ? __builtin_nontemporal_load(reinterpret_cast<const f32x4v *>(rp16 + e))
                                 : __builtin_nontemporal_load(reinterpret_cast<const f32x4v *>(rp32 + e));
    };
    auto unpack = [&](const f32x4v &u, float *xs) {
      if constexpr (IN == kInLogitsBf16) {
        const uint32_t wd[4] = {__float_as_uint(u.x), __float_as_uint(u.y), __float_as_uint(u.z),
                                __float_as_uint(u.w)};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          xs[2 * j] = bf16_to_f32(wd[j] & 0xffffu);
          xs[2 * j + 1] = __uint_as_float(wd[j] & 0xffff0000u);
        }
      } else {
        xs[0] = u.x;
        xs[1] = u.y;
        xs[2] = u.z;
        xs[3] = u.w;
      }
    };
    if (vec) {
      // The block reads one contiguous window of kLoads * 4 KB per
      // iteration: load u of wave w covers 1 KB chunk 4*u + w of the window.
      // One stream per segment (rather than one per wave) and non-temporal
      // loads (the rows are read once) keep HBM efficient when a thousand
      // segments stream at once.  One ballot tests the lane maxima of the
      // window against the threshold, and the normaliser takes the window
      // in one update.
      constexpr int step = EPL * kWave;             // elements per 1 KB chunk
      constexpr int win = kLoads * NW * step;       // elements per window
      // the window at base, its loads in r
      auto window = [&](int base, const f32x4v (&r)[kLoads]) {
        const int e = base + w * step + EPL * x;
        float xs[kLoads * EPL];
#pragma unroll
        for (int u = 0; u < kLoads; ++u) unpack(r[u], xs + u * EPL);
        float lmx[kLoads];
#pragma unroll
        for (int u = 0; u < kLoads; ++u) {
          lmx[u] = xs[u * EPL];
#pragma unroll
          for (int j = 1; j < EPL; ++j) lmx[u] = vmax(lmx[u], xs[u * EPL + j]);
        }
        float mx = lmx[0];
#pragma unroll
        for (int u = 1; u < kLoads; ++u) mx = vmax(mx, lmx[u]);
        if (base == lo) F.seed(mx);                 // the first window's lane maxima
        if (__ballot(mx >= F.thr_v) != 0ull) {
#pragma unroll
          for (int u = 0; u < kLoads; ++u)
            F.template offer<EPL, PIPE>(xs + u * EPL, lmx[u], e + u * NW * step, true);
        }
        if constexpr (LOGITS) nm.add(xs, mx, c2);
      };
      auto issue = [&](int base, f32x4v (&r)[kLoads]) {
        const int e = base + w * step + EPL * x;
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
      for (int e = base + w * step + EPL * x; e - EPL * x < hi; e += NW * step) {
        const bool in = e < hi;
        float xs[EPL];
        if (in) {
          unpack(load(e), xs);
        } else {
#pragma unroll
          for (int j = 0; j < EPL; ++j) xs[j] = -INFINITY;
        }
        float mx = xs[0];
#pragma unroll
        for (int j = 1; j < EPL; ++j) mx = vmax(mx, xs[j]);
        F.template offer<EPL, PIPE>(xs, mx, e, in);
        if constexpr (LOGITS) {
          if (in) nm.add(xs, mx, c2);
        }
      }
    } else {
      for (int e0 = lo + w * kWave; e0 < hi; e0 += NW * kWave) {
        const int e = e0 + x;
        const bool in = e < hi;
        float xs[1] = {-INFINITY};
        if (in) xs[0] = IN == kInLogitsBf16 ? bf16_to_f32(rp16[e]) : rp32[e];
        F.template offer<1, false>(xs, xs[0], e, in);
        if constexpr (LOGITS) {
          if (in) nm.add(xs, xs[0], c2);
        }
      }
    }
    F.fold();
    if constexpr (LOGITS) {
      // the wave's lanes in butterfly order, then the waves in order
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) {
        const float om = __shfl_xor(nm.m, off, kWave), os = __shfl_xor(nm.s, off, kWave);
        if (x & off) {
          Norm t;
          t.m = om;
          t.s = os;
          t.merge(nm.m, nm.s, c2);
          nm = t;
        } else {
          nm.merge(om, os, c2);
        }
      }
      if (x == 0) s_norm[w] = make_float2(nm.m, nm.s);
    }
    __syncthreads();

    // wave 0 merges the four per-wave lists: lane r < K holds the r-th best
    if (w == 0) {
      Norm tot;
      if constexpr (LOGITS) {
#pragma unroll
        for (int j = 0; j < NW; ++j) tot.merge(s_norm[j].x, s_norm[j].y, c2);
      }
      float bv;
      int bi;
      wave_best_k<K>(NW * K, [&](int c, float &v, int &i) {
        v = (&s_tv[0][0])[c];
        i = (&s_ti[0][0])[c];
      }, bv, bi);
      bool emit = lo == 0 && hi == V;                 // a whole row: no other segment
      bool late = false;
      if (!emit) {
        const int64_t trow = row - nwhole;            // the row among the cut ones
        const int64_t first = trow * V / per;         // pieces holding the row's first and last elements
        const int64_t last = (trow * V + V - 1) / per;
        const int nseg = static_cast<int>(last - first + 1);
        const int64_t s0 = trow * maxseg;
        const int64_t slot = s0 + (bid - nwhole - first);
        // publish the segment's list (lane r its r-th entry), then count
        // the segment on the row's counter: a relaxed count, since the
        // words carry their own flags
        if (x < K) put_word(part + slot * K + x, pack_entry(bv, bi));
        if (LOGITS && x == 0) put_word(part_n + slot, pack_norm(tot.m, tot.s));
        unsigned ticket = 0;
        if (x == 0) ticket = __hip_atomic_fetch_add(cnt + trow, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        ticket = __shfl(ticket, 0, kWave);
        if (ticket + 1 == static_cast<unsigned>(nseg)) {
          // the last segment: every other one has counted itself and its
          // words are on their way; read them as they land, then set them
          // and the counter back to zero for the next call
          unsigned long long *words = part + s0 * K;
          wave_best_k<K>(nseg * K, [&](int c, float &v, int &i) {
            const unsigned long long wd = await_word(words + c, wait_limit, late);
            v = __uint_as_float(static_cast<unsigned>(wd >> 32));
            i = static_cast<int>(static_cast<unsigned>(wd) - 1u);
          }, bv, bi);
          if constexpr (LOGITS) {
            tot = Norm();
            for (int j = 0; j < nseg; ++j) {
              const unsigned long long wd = await_word(part_n + s0 + j, wait_limit, late);
              tot.merge(__uint_as_float(static_cast<unsigned>(wd >> 32)), __uint_as_float(static_cast<unsigned>(wd)),
                        c2);
            }
          }
          for (int c = x; c < nseg * K; c += kWave) put_word(words + c, 0ull);
          if (LOGITS)
            for (int j = x; j < nseg; j += kWave) put_word(part_n + s0 + j, 0ull);
          if (x == 0) __hip_atomic_store(cnt + trow, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          late = __any(late);
          if (late && x == 0) raise_status(status, SDV_STATUS_TOPK_MERGE_WAIT);
          emit = true;
        }
      }
      if (emit && x < k) {
        const float pv = LOGITS ? __builtin_amdgcn_exp2f((bv - tot.m) * c2) / tot.s : bv;
        out_v[row * k + x] = late ? __builtin_nanf("") : pv;    // a published list never arrived
        out_i[row * k + x] = late ? -1 : bi;
      }
    }
    __syncthreads();                                  // the LDS lists are reused by the next segment
  };
  if (bid < nwhole) {
    segment(bid, 0, V);
    return;
  }
  // piece bid - nwhole of the cut rows: elements [t0, t1) counted from row nwhole
  const int64_t t0 = (bid - nwhole) * per;
  const int64_t t1 = min((rows - nwhole) * V, t0 + per);
  const int64_t r0 = t0 / V;
  segment(nwhole + r0, static_cast<int>(t0 - r0 * V), static_cast<int>(min<int64_t>(t1 - r0 * V, V)));
  if (t1 > (r0 + 1) * V) segment(nwhole + r0 + 1, 0, static_cast<int>(t1 - (r0 + 1) * V));
}

struct TopkPlan {
  int K;
  int64_t nwhole;    // rows scanned whole, one block each
  int64_t per;       // elements per piece of the other rows (0: none)
  int64_t blocks;
  int maxseg;        // segments per cut row at most
  int64_t cut;       // rows cut into pieces
};

// rows = q * CUs + r: the first q * CUs rows whole, the r others in pieces,
// one per CU (four per CU when q = 0), each at least a window and less than
// a row; a whole block per row when r = 0 or the pieces would not be
// shorter than a row, except that one to three rows per CU (r = 0) are all
// cut into row-aligned pieces when V allows.  Pieces cross row boundaries
// at most once.
constexpr int kTopkPiecesPerCuAlone = 4;

TopkPlan plan_topk(int64_t rows, int V, int k) {
  TopkPlan p;
  p.K = 1;
  while (p.K < k) p.K <<= 1;
  p.nwhole = rows;
  p.per = 0;
  p.blocks = rows;
  p.maxseg = 0;
  p.cut = 0;
  const int64_t cus = num_cus();
  const int64_t q = rows / cus, r = rows % cus;
  if (r == 0 && q > 0 && q < kTopkPiecesPerCuAlone && rows <= kTopkRowsMax) {
    // one to three rows per CU: every row in s equal pieces (four workgroups
    // per CU or more) when V splits into whole 16-byte loads, so that no
    // piece crosses a row boundary
    const int64_t sp = (kTopkPiecesPerCuAlone + q - 1) / q;
    if (V % (8 * sp) == 0 && V / sp >= 4096) {
      p.nwhole = 0;
      p.per = V / sp;
      p.cut = rows;
      p.blocks = rows * sp;
      p.maxseg = static_cast<int>((V - 1) / p.per + 2);
    }
    return p;
  }
  if (r == 0 || r > kTopkRowsMax) return p;
  const int64_t tail = r * static_cast<int64_t>(V);
  const int64_t pieces = (q == 0 ? kTopkPiecesPerCuAlone : 1) * cus;
  int64_t per = (tail + pieces - 1) / pieces;
  per = (per + 7) / 8 * 8;                            // whole 16-byte loads of fp32 and bf16
  if (per < 4096) per = 4096;                         // at least a window (fp32) per piece
  if (per >= V) return p;
  p.nwhole = q * cus;
  p.per = per;
  p.cut = r;
  p.blocks = p.nwhole + (tail + per - 1) / per;
  p.maxseg = static_cast<int>((V - 1) / per + 2);
  return p;
}

size_t topk_workspace(int64_t rows, int V, int k, bool logits) {
  const TopkPlan p = plan_topk(rows, V, k);
  if (p.per == 0) return 0;
  Carver c(nullptr);
  c.take<char>(kWsHeaderBytes);
  c.take<unsigned>(kTopkRowsMax);
  c.take<unsigned long long>(static_cast<size_t>(p.cut) * p.maxseg * p.K);
  if (logits) c.take<unsigned long long>(static_cast<size_t>(p.cut) * p.maxseg);
  return c.bytes();
}

template <int K, int IN>
int32_t launch_topk(const void *rows_in, int64_t rows, int V, int k, const TopkPlan &p, bool vec, float c2,
                    float *out_v, int *out_i, unsigned *cnt, unsigned long long *part,
                    unsigned long long *part_n, unsigned *status, hipStream_t st) {
  hipLaunchKernelGGL((topk_kernel<K, IN>), dim3(static_cast<unsigned>(p.blocks)), dim3(kTopkThreads), 0, st,
                     rows_in, rows, V, p.nwhole, p.per, p.maxseg, k, vec, c2, out_v, out_i, cnt, part, part_n,
                     status, wait_limit(kTopkSpin));
  return check_launch("topk_kernel");
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
  unsigned *cnt = nullptr, *status = nullptr;
  unsigned long long *part = nullptr, *part_n = nullptr;
  if (p.per > 0) {
    Carver c(ws);
    status = reinterpret_cast<unsigned *>(c.take<char>(kWsHeaderBytes)) + kWsStatus;
    cnt = c.take<unsigned>(kTopkRowsMax);
    part = c.take<unsigned long long>(static_cast<size_t>(p.cut) * p.maxseg * p.K);
    if (IN != kInProbs) part_n = c.take<unsigned long long>(static_cast<size_t>(p.cut) * p.maxseg);
  }
  const int epl = IN == kInLogitsBf16 ? 8 : 4;
  const bool vec = (V % epl == 0) && (reinterpret_cast<uintptr_t>(rows_in) % 16 == 0);
  hipStream_t st = as_stream(stream);
#define SDV_TOPK_IN(KK)                                                                                          \
  (IN == kInProbs        ? launch_topk<KK, kInProbs>(rows_in, rows, V, k, p, vec, c2, topk_p, topk_id, cnt, part, \
                                                     part_n, status, st)                                         \
   : IN == kInLogitsF32 ? launch_topk<KK, kInLogitsF32>(rows_in, rows, V, k, p, vec, c2, topk_p, topk_id, cnt, part, \
                                                         part_n, status, st)                                     \
                         : launch_topk<KK, kInLogitsBf16>(rows_in, rows, V, k, p, vec, c2, topk_p, topk_id, cnt, part, \
                                                          part_n, status, st))
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
