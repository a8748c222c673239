// A2-A4: candidate tree from the per-step top-k ("[SGLang] Multi-Layer
// EAGLE" section 2, select_top_k_tokens / tree_info; build_eagle_tree in
// "EAGLE speculative decoding in four parts", "Drafting, verification and
// slots"), plus positions, the tree mask and the retrieve arrays
// (zero-to-sglang ch.10 section 5.2).
//
// Latency-bound integer work: one 1024-thread block per request keeps its
// top-k lists and the whole candidate pool in LDS.  Every selection (each
// step's frontier and the final best N-1) follows the strict order (score
// desc, pool index asc) of 64-bit order keys, so the result is deterministic.
// When a step's k*k candidates fit one wave (k <= 8), wave 0 runs the steps
// with sorting networks in registers and, for N - 1 <= 64, keeps the running
// best 64; otherwise a selection is a rank computation over the block (an
// entry's rank is the number of entries that beat it).  The per-node arrays
// (first child, next sibling, mask rows) then take all waves, a group of
// lanes per node.
#include <climits>

#include "common.hpp"

namespace sdv {
namespace {

constexpr int kTreeThreads = 1024;
constexpr int kTreeWaves = kTreeThreads / kWave;
constexpr int kMaxPool = 2048;
constexpr int kMaxNodes = 256;
constexpr int kMaxWords = kMaxNodes / 32;

// Order key of pool entry e: larger key = better under (score desc, pool
// index asc).  The score's bits are mapped to an unsigned order (-0 is
// folded into +0 first, so equal scores still tie on the index).
__device__ __forceinline__ unsigned long long order_key(float score, int e) {
  const unsigned u = __float_as_uint(score + 0.0f);
  const unsigned su = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return (static_cast<unsigned long long>(su) << 32) | static_cast<unsigned>(~e);
}

// The score a key was made from (a -0 score comes back as +0).
__device__ __forceinline__ float score_of_key(unsigned long long key) {
  const unsigned su = static_cast<unsigned>(key >> 32);
  return __uint_as_float((su & 0x80000000u) ? (su & 0x7FFFFFFFu) : ~su);
}

// Ranks the n entries [lo, lo + n) among themselves (rank = how many beat
// it).  g lanes share an entry (g a power of two, g * n <= threads, g <= 64)
// and split its comparisons; f(e, rank) is called by the group's first lane.
template <typename F>
__device__ __forceinline__ void rank_block(const unsigned long long *key, int lo, int n, F f) {
  int g = 1;
  while (g < kWave && 2 * g * n <= kTreeThreads) g <<= 1;
  const int per_pass = kTreeThreads / g;
  for (int ent0 = 0; ent0 < n; ent0 += per_pass) {
    const int ent = ent0 + static_cast<int>(threadIdx.x) / g, part = static_cast<int>(threadIdx.x) % g;
    int r = 0;
    if (ent < n) {
      const unsigned long long ke = key[lo + ent];
#pragma unroll 16
      for (int o = lo + part; o < lo + n; o += g) r += key[o] > ke;
    }
    for (int off = 1; off < g; off <<= 1) r += __shfl_xor(r, off, kWave);
    if (ent < n && part == 0) f(lo + ent, r);
  }
}

// Lane l's value of lane l ^ S, without LDS: DPP for S <= 8, the row-half
// swaps for 16 and 32.  Where the builtin's direction could be either
// (row shifts; which swap output is the partner's), the same instruction
// moves the lane ids and the copy that came from lane l ^ S is taken.
template <int S>
__device__ __forceinline__ unsigned xor_lane(unsigned v, unsigned lane) {
  if constexpr (S == 1) {
    return static_cast<unsigned>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0xB1, 0xF, 0xF, true));   // quad [1,0,3,2]
  } else if constexpr (S == 2) {
    return static_cast<unsigned>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0x4E, 0xF, 0xF, true));   // quad [2,3,0,1]
  } else if constexpr (S == 4) {
    const unsigned a = static_cast<unsigned>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0x104, 0xF, 0xF, true));
    const unsigned b = static_cast<unsigned>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0x114, 0xF, 0xF, true));
    const unsigned la = static_cast<unsigned>(__builtin_amdgcn_mov_dpp(static_cast<int>(lane), 0x104, 0xF, 0xF, true));
    return la == (lane ^ 4u) ? a : b;                                                                     // row shifts by 4
  } else if constexpr (S == 8) {
    return static_cast<unsigned>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0x128, 0xF, 0xF, true));  // row rotate by 8
  } else if constexpr (S == 16) {
    const auto p = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    const auto q = __builtin_amdgcn_permlane16_swap(lane, lane, false, false);
    return q[0] == (lane ^ 16u) ? p[0] : p[1];
  } else {
    const auto p = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    const auto q = __builtin_amdgcn_permlane32_swap(lane, lane, false, false);
    return q[0] == (lane ^ 32u) ? p[0] : p[1];
  }
}

template <int S>
__device__ __forceinline__ unsigned long long xor_lane64(unsigned long long v, unsigned lane) {
  const unsigned lo = xor_lane<S>(static_cast<unsigned>(v), lane);
  const unsigned hi = xor_lane<S>(static_cast<unsigned>(v >> 32), lane);
  return (static_cast<unsigned long long>(hi) << 32) | lo;
}

// One move of a 64-bit value across the wave by a DPP pattern.
template <int CTRL>
__device__ __forceinline__ unsigned long long dpp64(unsigned long long v) {
  const int lo = __builtin_amdgcn_mov_dpp(static_cast<int>(v), CTRL, 0xF, 0xF, true);
  const int hi = __builtin_amdgcn_mov_dpp(static_cast<int>(v >> 32), CTRL, 0xF, 0xF, true);
  return (static_cast<unsigned long long>(static_cast<unsigned>(hi)) << 32) | static_cast<unsigned>(lo);
}

// Lane l's value of lane l ^ (SIZE - 1): the mirror image within aligned
// blocks of SIZE lanes (quad and row mirrors by DPP, then the row-half swaps).
template <int SIZE>
__device__ __forceinline__ unsigned long long mirror64(unsigned long long v, unsigned lane) {
  if constexpr (SIZE == 2) {
    return xor_lane64<1>(v, lane);
  } else if constexpr (SIZE == 4) {
    return dpp64<0x1B>(v);                                        // quad [3,2,1,0]
  } else if constexpr (SIZE == 8) {
    return dpp64<0x141>(v);                                       // half-row mirror
  } else if constexpr (SIZE == 16) {
    return dpp64<0x140>(v);                                       // row mirror
  } else if constexpr (SIZE == 32) {
    return xor_lane64<16>(dpp64<0x140>(v), lane);
  } else {
    return xor_lane64<32>(xor_lane64<16>(dpp64<0x140>(v), lane), lane);
  }
}

// Compare-exchange with the lane at stride S: within each pair the lower
// lane keeps the larger key when DESC, the smaller otherwise.  One
// comparison decides both lanes (equal keys, only the zero fill, swap
// harmlessly).
template <int S, bool DESC>
__device__ __forceinline__ unsigned long long half_stage(unsigned long long key, unsigned lane) {
  const unsigned long long other = xor_lane64<S>(key, lane);
  const bool keep_max = ((lane & S) == 0) == DESC;
  return (other > key) == keep_max ? other : key;
}

// Half-cleaners at strides S, S/2, .., 1: sort every aligned block of 2S
// lanes that holds a bitonic sequence.
template <int S, bool DESC>
__device__ __forceinline__ unsigned long long cleaners(unsigned long long key, unsigned lane) {
  if constexpr (S >= 1) {
    key = half_stage<S, DESC>(key, lane);
    return cleaners<S / 2, DESC>(key, lane);
  } else {
    return key;
  }
}

// Sorts largest first, assuming every aligned block of LO / 2 lanes already
// is: the levels LO, 2 LO, .., HI each merge two sorted halves of a block by
// comparing every lane of the lower half with its mirror image in the upper
// half (lower keeps the larger) and then sorting both bitonic halves.  Lanes
// past HI must already be in order with the rest (zero fill).
template <int LO, int HI>
__device__ __forceinline__ unsigned long long merge_sort_desc(unsigned long long key, unsigned lane) {
  if constexpr (LO <= HI) {
    const unsigned long long other = mirror64<LO>(key, lane);
    const bool keep_max = (lane & (LO / 2)) == 0;
    key = (other > key) == keep_max ? other : key;
    key = cleaners<LO / 4, true>(key, lane);
    return merge_sort_desc<LO * 2, HI>(key, lane);
  } else {
    return key;
  }
}

// Largest 64 of a (lane-sorted smallest first) and b (largest first),
// smallest first: the lane-wise maxima form a bitonic sequence that holds
// the top 64, and the six half-cleaner stages of a 64-lane merge sort it.
__device__ __forceinline__ unsigned long long merge_top_asc(unsigned long long a, unsigned long long b,
                                                             unsigned lane) {
  return cleaners<32, false>(a > b ? a : b, lane);
}

// Minimum over aligned groups of g lanes (g a power of two, at most 64,
// uniform across the wave, every lane active).
__device__ __forceinline__ unsigned group_min(unsigned v, int g, unsigned lane) {
  if (g > 1) v = min(v, xor_lane<1>(v, lane));
  if (g > 2) v = min(v, xor_lane<2>(v, lane));
  if (g > 4) v = min(v, xor_lane<4>(v, lane));
  if (g > 8) v = min(v, xor_lane<8>(v, lane));
  if (g > 16) v = min(v, xor_lane<16>(v, lane));
  if (g > 32) v = min(v, xor_lane<32>(v, lane));
  return v;
}

__device__ __forceinline__ int entry_of_key(unsigned long long key) {
  return static_cast<int>(~static_cast<unsigned>(key));
}

// Exclusive block scan of one int per thread.
__device__ int block_exclusive_scan(int x) {
  __shared__ int s_w[kTreeWaves];
  const int l = lane_id(), w = threadIdx.x / kWave;
  int inc = x;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int y = __shfl_up(inc, off, kWave);
    if (l >= off) inc += y;
  }
  if (l == kWave - 1) s_w[w] = inc;
  __syncthreads();
  int before = 0;
  for (int j = 0; j < w; ++j) before += s_w[j];
  __syncthreads();
  return before + inc - x;
}

// The draft steps in wave 0 when every step's k*k candidates fit one wave
// (k <= 8).  Candidate c of frontier slot j sits in lane j * K2 + c (K2 = k
// rounded up to a power of two; lanes without a candidate hold key 0, below
// every key).  With RUNS (every top-k row sorted largest first, entries in
// [0, 1]) each slot's children are already in order -- their scores are one
// non-negative factor times a falling sequence and ties go to the smaller
// pool index -- so each step's sort starts from runs of K2; otherwise it
// sorts from scratch.  Each step's keys end largest first (frontier slot j
// in lane j).  With FINAL the best 64 keys of the pool so far are kept
// smallest first and every step's keys merge into them one step late, in
// the same straight-line code as the next step's sort.  The candidates'
// scores, parents, keys and the frontier's draft rows go to LDS; a frontier
// entry's score comes back from its key.
template <int K2, bool RUNS, bool FINAL>
__device__ unsigned long long wave_steps(int k, int S, const float *s_tp, float *s_score, int *s_par,
                                         unsigned long long *s_key, int *s_row) {
  constexpr int LO = RUNS ? 2 * K2 : 2;
  const int x = static_cast<int>(threadIdx.x);
  const unsigned lane = static_cast<unsigned>(x);
  unsigned long long key = 0;
  if (x < k) {                      // step 0: the root's children
    key = order_key(s_tp[x], x);
    s_score[x] = s_tp[x];
    s_par[x] = -1;
    s_key[x] = key;
  }
  key = merge_sort_desc<LO, RUNS ? K2 : kWave>(key, lane);
  unsigned long long best = 0, pend = key;
  const int j = x / K2, c = x % K2;   // the frontier slot and child this lane expands
  for (int i = 1; i < S; ++i) {
    if (x < k) s_row[entry_of_key(key)] = 1 + (i - 1) * k + x;
    const unsigned long long fk = __shfl(key, j, kWave);
    unsigned long long ck = 0;
    if (j < k && c < k) {
      const int e = k + (i - 1) * k * k + j * k + c;
      const float sc = score_of_key(fk) * s_tp[e];
      s_score[e] = sc;
      s_par[e] = entry_of_key(fk);
      ck = order_key(sc, e);
      s_key[e] = ck;
    }
    key = merge_sort_desc<LO, RUNS ? K2 * K2 : kWave>(ck, lane);
    if constexpr (FINAL) best = merge_top_asc(best, pend, lane);
    pend = key;
  }
  if constexpr (FINAL) best = merge_top_asc(best, pend, lane);
  return best;
}



// Pool entry e of a request coincides with entry e of its row-major [R, k]
// top-k lists: step 0 holds the root's k children (row 0), and entry
// k + (i-1)*k*k + j*k + c of step i >= 1 is child c of frontier slot j,
// drawn from row 1 + (i-1)*k + j.
// K2 = 0: a step's candidates do not fit one wave (k > 8); otherwise K2 is
// k rounded up to a power of two and FINAL says N - 1 <= 64.  The host picks
// both from the shape, so each kernel holds only its own two forms of the
// steps, sorted runs or not (one kernel with all ten forms took 0.4 us
// longer over the c3 steps).
template <int K2, bool FINAL>
__global__ void __launch_bounds__(kTreeThreads)
build_tree_kernel(int k, int S, int N, const float *__restrict__ topk_p,
                  const int *__restrict__ topk_id, const int *__restrict__ root_token,
                  const int *__restrict__ prefix_len, int *__restrict__ o_tokens,
                  int *__restrict__ o_parent, int *__restrict__ o_depth,
                  int *__restrict__ o_positions, float *__restrict__ o_score,
                  int *__restrict__ o_qrow, uint8_t *__restrict__ o_mask,
                  uint32_t *__restrict__ o_bits, int *__restrict__ o_retrieve,
                  int *__restrict__ o_next_token, int *__restrict__ o_next_sibling) {
  extern __shared__ unsigned char smem[];
  const int M = k + (S - 1) * k * k;
  unsigned long long *s_key = reinterpret_cast<unsigned long long *>(smem);
  float *s_tp = reinterpret_cast<float *>(s_key + M);
  int *s_tok = reinterpret_cast<int *>(s_tp + M);
  float *s_score = reinterpret_cast<float *>(s_tok + M);
  int *s_par = reinterpret_cast<int *>(s_score + M);   // pool index of the parent, -1 = root
  int *s_row = s_par + M;                                // draft row of the entry's children, -1
  int *s_tree = s_row + M;                               // tree index, -1 if not selected
  __shared__ int s_front[32];
  __shared__ int s_tpar[kMaxNodes];
  __shared__ __align__(16) int s_sel[kWave];
  __shared__ int s_bad[kTreeWaves];

  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const float *tp = topk_p + static_cast<int64_t>(b) * M;
  const int *ti = topk_id + static_cast<int64_t>(b) * M;
  bool runs = true;                  // every top-k row falls, entries in [0, 1]
  for (int e = tid; e < M; e += kTreeThreads) {
    const float v = tp[e];
    s_tp[e] = v;
    s_tok[e] = ti[e];
    s_row[e] = -1;
    s_tree[e] = -1;
    runs = runs && v >= 0.0f && v <= 1.0f && ((e + 1) % k == 0 || v >= tp[e + 1]);   // rows are blocks of k
  }
  const unsigned long long bad = __ballot(!runs);
  if (lane_id() == 0) s_bad[tid / kWave] = bad != 0;
  const int L = prefix_len[b];
  const int root = root_token[b];
  const int64_t ob = static_cast<int64_t>(b) * N;
  if (tid == 0) {
    o_tokens[ob] = root;
    o_parent[ob] = -1;
    o_depth[ob] = 0;
    o_positions[ob] = L;
    o_score[ob] = 1.0f;
    o_qrow[ob] = 0;
    s_tpar[0] = -1;
  }
  __syncthreads();

  // With N - 1 <= 64 as well, wave 0 also keeps the best 64 keys of the
  // pool so far (every step's sorted keys merged in) and then numbers and
  // writes the final N - 1 itself.
  constexpr bool wave_final = FINAL;
  if constexpr (K2 > 0) {
    if (tid < kWave) {
      const int x = tid;
      runs = true;
#pragma unroll
      for (int w = 0; w < kTreeWaves; ++w) runs = runs && !s_bad[w];
      const unsigned long long best = runs ? wave_steps<K2, true, FINAL>(k, S, s_tp, s_score, s_par, s_key, s_row)
                                           : wave_steps<8, false, FINAL>(k, S, s_tp, s_score, s_par, s_key, s_row);
      if constexpr (FINAL) {
        // lanes 65 - N .. 63 hold the best N - 1 entries; an entry's tree
        // index is 1 + the number of the others with a smaller pool index.
        // The LDS writes of this wave land before its later reads.
        const bool sel = x >= kWave - (N - 1);
        const int e = sel ? entry_of_key(best) : INT_MAX;
        s_sel[x] = e;
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
        int below = 0;
#pragma unroll
        for (int y = 0; y < kWave; y += 4) {
          const int4 v = *reinterpret_cast<const int4 *>(&s_sel[y]);
          below += (v.x < e) + (v.y < e) + (v.z < e) + (v.w < e);
        }
        const int te = 1 + below;
        if (sel) s_tree[e] = te;
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
        if (sel) {
          const int pe = s_par[e];
          const int tpar = pe < 0 ? 0 : s_tree[pe];   // -1 only if scores broke monotonicity
          const int step = e < k ? 0 : 1 + (e - k) / (k * k);
          o_tokens[ob + te] = s_tok[e];
          o_parent[ob + te] = tpar;
          o_depth[ob + te] = step + 1;
          o_positions[ob + te] = L + step + 1;
          o_score[ob + te] = s_score[e];
          o_qrow[ob + te] = s_row[e];
          s_tpar[te] = tpar;
        }
      }
    }
    __syncthreads();
  } else {
    // step 0: the root's children; their rank order is the first frontier
    for (int c = tid; c < k; c += kTreeThreads) {
      s_score[c] = s_tp[c];
      s_par[c] = -1;
      s_key[c] = order_key(s_tp[c], c);
    }
    __syncthreads();
    rank_block(s_key, 0, k, [&](int e, int r) { s_front[r] = e; });
    __syncthreads();

    // steps 1 .. S-1: expand every frontier slot, keep the best k as the next frontier
    for (int i = 1; i < S; ++i) {
      const int base = k + (i - 1) * k * k;
      for (int x = tid; x < k * k; x += kTreeThreads) {
        const int f = s_front[x / k];
        const int e = base + x;
        const float sc = s_score[f] * s_tp[e];
        s_score[e] = sc;
        s_par[e] = f;
        s_key[e] = order_key(sc, e);
      }
      for (int j = tid; j < k; j += kTreeThreads) s_row[s_front[j]] = 1 + (i - 1) * k + j;
      __syncthreads();
      rank_block(s_key, base, k * k, [&](int e, int r) {
        if (r < k) s_front[r] = e;
      });
      __syncthreads();
    }
  }

  // final selection by ranks over the whole pool: the best N-1 entries,
  // numbered in pool order
  if constexpr (!wave_final) {
    rank_block(s_key, 0, M, [&](int e, int r) { s_tree[e] = r < N - 1 ? 1 : 0; });
    __syncthreads();
    const int per = (M + kTreeThreads - 1) / kTreeThreads;
    const int e0 = tid * per;
    int cnt = 0;
    for (int e = e0; e < min(M, e0 + per); ++e) cnt += s_tree[e];
    int t = 1 + block_exclusive_scan(cnt);   // tree index of this thread's first selected entry
    for (int e = e0; e < min(M, e0 + per); ++e) s_tree[e] = s_tree[e] ? t++ : -1;
    __syncthreads();
    for (int e = tid; e < M; e += kTreeThreads) {
      const int te = s_tree[e];
      if (te < 0) continue;
      const int pe = s_par[e];
      const int tpar = pe < 0 ? 0 : s_tree[pe];   // -1 only if scores broke monotonicity
      const int step = e < k ? 0 : 1 + (e - k) / (k * k);
      o_tokens[ob + te] = s_tok[e];
      o_parent[ob + te] = tpar;
      o_depth[ob + te] = step + 1;
      o_positions[ob + te] = L + step + 1;
      o_score[ob + te] = s_score[e];
      o_qrow[ob + te] = s_row[e];
      s_tpar[te] = tpar;
    }
    __syncthreads();
  }

  // ---- per node, g lanes each (g a power of two, at most 64, g * N <= the
  // block): the first child and next sibling (the smallest larger index with
  // the node as parent / with the same parent), the ancestor bits (the mask
  // row) and the retrieve index.  A group lies inside one wave.
  int lg = 0;
  while (lg < 6 && (2 << lg) * N <= kTreeThreads) ++lg;
  const int g = 1 << lg;
  const int n = tid >> lg, part = tid & (g - 1);
  const unsigned lane = static_cast<unsigned>(lane_id());
  const bool live = n < N;
  const int p = live ? s_tpar[n] : -1;
  unsigned fc = UINT_MAX, ns = UINT_MAX;
  if (live) {
    for (int m = n + 1 + part; m < N; m += g) {
      const int pm = s_tpar[m];
      if (pm == n) fc = min(fc, static_cast<unsigned>(m));
      if (p >= 0 && pm == p) ns = min(ns, static_cast<unsigned>(m));
    }
  }
  fc = group_min(fc, g, lane);
  ns = group_min(ns, g, lane);
  uint32_t bits[kMaxWords];
#pragma unroll
  for (int w = 0; w < kMaxWords; ++w) bits[w] = 0;
  int j = live ? n : -1;
  for (int hop = 0; hop <= S && j >= 0; ++hop) {
#pragma unroll
    for (int w = 0; w < kMaxWords; ++w)
      if (w == j / 32) bits[w] |= 1u << (j % 32);
    j = s_tpar[j];
  }
  auto word = [&](int wi) {
    uint32_t r = 0;
#pragma unroll
    for (int w = 0; w < kMaxWords; ++w)
      if (w == wi) r = bits[w];
    return r;
  };
  if (live) {
    const int64_t row = ob + n;
    if (part == 0) {
      o_next_token[row] = fc == UINT_MAX ? -1 : static_cast<int>(fc);
      o_next_sibling[row] = ns == UINT_MAX ? -1 : static_cast<int>(ns);
      o_retrieve[row] = static_cast<int>(row);
    }
    const int W = (N + 31) / 32;
    if (o_bits)
      for (int w = part; w < W; w += g) o_bits[row * W + w] = word(w);
    if (o_mask) {
      uint8_t *mrow = o_mask + row * N;
      if (N % 4 == 0 && (reinterpret_cast<uintptr_t>(o_mask) & 3) == 0) {
        // four columns per store: bit c of the row -> byte c
        for (int q = part; 4 * q < N; q += g) {
          const uint32_t nib = (word(q / 8) >> (4 * (q % 8))) & 0xFu;
          reinterpret_cast<uint32_t *>(mrow)[q] =
              (nib & 1u) | ((nib & 2u) << 7) | ((nib & 4u) << 14) | ((nib & 8u) << 21);
        }
      } else {
        for (int c = part; c < N; c += g) mrow[c] = static_cast<uint8_t>((word(c / 32) >> (c % 32)) & 1u);
      }
    }
  }
}

// Multi-layer draft chain ("[SGLang] Multi-Layer EAGLE", sections 2-3: one
// draft layer per step, the per-step top-1 lists concatenated, step i's
// parent the token of step i-1): every output is closed-form, so one
// 256-thread block per request writes them, thread i for node i (and mask
// row i).
constexpr int kChainThreads = 256;

__global__ void __launch_bounds__(kChainThreads)
build_chain_kernel(int S, const float *__restrict__ topk_p, const int32_t *__restrict__ topk_id,
                   const int32_t *__restrict__ root_token, const int32_t *__restrict__ prefix_len,
                   int32_t *__restrict__ tokens, int32_t *__restrict__ parent, int32_t *__restrict__ depth,
                   int32_t *__restrict__ positions, float *__restrict__ score, int32_t *__restrict__ q_row,
                   uint8_t *__restrict__ mask, uint32_t *__restrict__ mask_bits,
                   int32_t *__restrict__ retrieve_index, int32_t *__restrict__ next_token,
                   int32_t *__restrict__ next_sibling) {
  const int b = blockIdx.x;
  const int N = S + 1;
  const int W = (N + 31) / 32;
  const int64_t o = static_cast<int64_t>(b) * N;
  for (int i = threadIdx.x; i < N; i += kChainThreads) {
    tokens[o + i] = i == 0 ? root_token[b] : topk_id[static_cast<int64_t>(b) * S + i - 1];
    parent[o + i] = i - 1;
    depth[o + i] = i;
    positions[o + i] = prefix_len[b] + i;
    score[o + i] = i == 0 ? 1.0f : topk_p[static_cast<int64_t>(b) * S + i - 1];
    q_row[o + i] = i < S ? i : -1;
    retrieve_index[o + i] = static_cast<int32_t>(o + i);
    next_token[o + i] = i < S ? i + 1 : -1;
    next_sibling[o + i] = -1;
    if (mask) {
      uint8_t *row = mask + (o + i) * N;
      for (int j = 0; j < N; ++j) row[j] = j <= i ? 1 : 0;
    }
    if (mask_bits) {
      uint32_t *row = mask_bits + (o + i) * W;
      for (int w = 0; w < W; ++w) {
        const int full = i + 1 - 32 * w;     // columns 32w .. i are set
        row[w] = full >= 32 ? 0xFFFFFFFFu : (full <= 0 ? 0u : (1u << full) - 1u);
      }
    }
  }
}

}  // namespace
}  // namespace sdv

using namespace sdv;

extern "C" int32_t sdv_build_tree(sdv_tree_shape sh, const float *topk_p, const int32_t *topk_id,
                                  const int32_t *root_token, const int32_t *prefix_len,
                                  int32_t *tokens, int32_t *parent, int32_t *depth,
                                  int32_t *positions, float *score, int32_t *q_row, uint8_t *mask,
                                  uint32_t *mask_bits, int32_t *retrieve_index,
                                  int32_t *retrieve_next_token, int32_t *retrieve_next_sibling,
                                  void *stream) {
  clear_error();
  SDV_REQUIRE(sh.B >= 0 && sh.k >= 1 && sh.S >= 1 && sh.N >= 1, SDV_E_SHAPE,
              "build_tree: need B >= 0, k >= 1, S >= 1, N >= 1");
  SDV_REQUIRE(sh.k <= 32, SDV_E_UNSUPPORTED, "build_tree: k=%d above 32", sh.k);
  const int64_t M = sh.k + static_cast<int64_t>(sh.S - 1) * sh.k * sh.k;
  SDV_REQUIRE(M <= kMaxPool, SDV_E_UNSUPPORTED, "build_tree: pool of %lld above %d",
              static_cast<long long>(M), kMaxPool);
  SDV_REQUIRE(sh.N - 1 <= M, SDV_E_SHAPE, "build_tree: N-1=%d exceeds the pool size %lld", sh.N - 1,
              static_cast<long long>(M));
  SDV_REQUIRE(sh.N <= kMaxNodes, SDV_E_UNSUPPORTED, "build_tree: N=%d above %d", sh.N, kMaxNodes);
  if (sh.B == 0) return SDV_OK;
  SDV_REQUIRE(topk_p && topk_id && root_token && prefix_len && tokens && parent && depth && positions &&
                  score && q_row && retrieve_index && retrieve_next_token && retrieve_next_sibling,
              SDV_E_NULL, "build_tree: NULL pointer");
  const size_t lds = static_cast<size_t>(M) * (6 * sizeof(int) + sizeof(uint64_t));   // key, tp, tok, score, par, row, tree
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3(sh.B), dim3(kTreeThreads), lds, as_stream(stream), sh.k, sh.S, sh.N, topk_p,
                       topk_id, root_token, prefix_len, tokens, parent, depth, positions, score, q_row, mask,
                       mask_bits, retrieve_index, retrieve_next_token, retrieve_next_sibling);
  };
  const bool fin = sh.N - 1 <= kWave;
  if (sh.k * sh.k > kWave) go(build_tree_kernel<0, false>);
  else if (sh.k == 1) fin ? go(build_tree_kernel<1, true>) : go(build_tree_kernel<1, false>);
  else if (sh.k == 2) fin ? go(build_tree_kernel<2, true>) : go(build_tree_kernel<2, false>);
  else if (sh.k <= 4) fin ? go(build_tree_kernel<4, true>) : go(build_tree_kernel<4, false>);
  else fin ? go(build_tree_kernel<8, true>) : go(build_tree_kernel<8, false>);
  return check_launch("build_tree_kernel");
}

extern "C" int32_t sdv_build_chain(int32_t B, int32_t S, const float *topk_p, const int32_t *topk_id,
                                   const int32_t *root_token, const int32_t *prefix_len, int32_t *tokens,
                                   int32_t *parent, int32_t *depth, int32_t *positions, float *score,
                                   int32_t *q_row, uint8_t *mask, uint32_t *mask_bits, int32_t *retrieve_index,
                                   int32_t *retrieve_next_token, int32_t *retrieve_next_sibling, void *stream) {
  clear_error();
  SDV_REQUIRE(B >= 0 && S >= 1, SDV_E_SHAPE, "build_chain: need B >= 0 and S >= 1");
  SDV_REQUIRE(S + 1 <= kMaxNodes, SDV_E_UNSUPPORTED, "build_chain: N=%d above %d", S + 1, kMaxNodes);
  if (B == 0) return SDV_OK;
  SDV_REQUIRE(topk_p && topk_id && root_token && prefix_len && tokens && parent && depth && positions &&
                  score && q_row && retrieve_index && retrieve_next_token && retrieve_next_sibling,
              SDV_E_NULL, "build_chain: NULL pointer");
  hipLaunchKernelGGL(build_chain_kernel, dim3(B), dim3(kChainThreads), 0, as_stream(stream), S, topk_p, topk_id,
                     root_token, prefix_len, tokens, parent, depth, positions, score, q_row, mask, mask_bits,
                     retrieve_index, retrieve_next_token, retrieve_next_sibling);
  return check_launch("build_chain_kernel");
}
