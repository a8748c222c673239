// A2-A4: candidate tree from the per-step top-k ("[SGLang] Multi-Layer
// EAGLE" section 2, select_top_k_tokens / tree_info; build_eagle_tree in
// "EAGLE speculative decoding in four parts", "Drafting, verification and
// slots"), plus positions, the tree mask and the retrieve arrays
// (zero-to-sglang ch.10 section 5.2).
//
// Latency-bound integer work: one 1024-thread block per request keeps its
// top-k lists and the whole candidate pool in LDS.  Every selection (each step's frontier and the
// final best N-1) is a rank computation under the strict order
// (score desc, pool index asc): an entry's rank is the number of entries that
// beat it, so ranks are unique and the result is deterministic.
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

// One bitonic stage of block size SIZE and stride S, larger keys first.
template <int SIZE, int S>
__device__ __forceinline__ unsigned long long sort_stage(unsigned long long key, unsigned lane) {
  const unsigned long long other = xor_lane64<S>(key, lane);
  const bool desc = (lane & SIZE) == 0;          // this block's direction
  const bool lower = (lane & S) == 0;            // this lane's place in the pair
  const bool keep_max = lower == desc;
  return keep_max ? (other > key ? other : key) : (other < key ? other : key);
}

// Sorts one order key per lane across the wave, largest first (a bitonic
// network of 21 compare-exchange stages, all in registers).
__device__ __forceinline__ unsigned long long wave_sort_keys_desc(unsigned long long key) {
  const unsigned lane = static_cast<unsigned>(lane_id());
  key = sort_stage<2, 1>(key, lane);
  key = sort_stage<4, 2>(key, lane);
  key = sort_stage<4, 1>(key, lane);
  key = sort_stage<8, 4>(key, lane);
  key = sort_stage<8, 2>(key, lane);
  key = sort_stage<8, 1>(key, lane);
  key = sort_stage<16, 8>(key, lane);
  key = sort_stage<16, 4>(key, lane);
  key = sort_stage<16, 2>(key, lane);
  key = sort_stage<16, 1>(key, lane);
  key = sort_stage<32, 16>(key, lane);
  key = sort_stage<32, 8>(key, lane);
  key = sort_stage<32, 4>(key, lane);
  key = sort_stage<32, 2>(key, lane);
  key = sort_stage<32, 1>(key, lane);
  key = sort_stage<64, 32>(key, lane);
  key = sort_stage<64, 16>(key, lane);
  key = sort_stage<64, 8>(key, lane);
  key = sort_stage<64, 4>(key, lane);
  key = sort_stage<64, 2>(key, lane);
  key = sort_stage<64, 1>(key, lane);
  return key;
}

// Largest 64 of two lane-sorted key sets (largest first), largest first:
// b reversed across the wave (lane l ^ 63) against a, the larger of each
// pair (a bitonic sequence holding the top 64), then the last six stages.
__device__ __forceinline__ unsigned long long wave_merge_top(unsigned long long a, unsigned long long b) {
  const unsigned lane = static_cast<unsigned>(lane_id());
  b = xor_lane64<32>(b, lane);
  b = xor_lane64<16>(b, lane);
  b = xor_lane64<8>(b, lane);
  b = xor_lane64<4>(b, lane);
  b = xor_lane64<2>(b, lane);
  b = xor_lane64<1>(b, lane);
  unsigned long long key = a > b ? a : b;
  key = sort_stage<64, 32>(key, lane);
  key = sort_stage<64, 16>(key, lane);
  key = sort_stage<64, 8>(key, lane);
  key = sort_stage<64, 4>(key, lane);
  key = sort_stage<64, 2>(key, lane);
  key = sort_stage<64, 1>(key, lane);
  return key;
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

// Pool entry e of a request coincides with entry e of its row-major [R, k]
// top-k lists: step 0 holds the root's k children (row 0), and entry
// k + (i-1)*k*k + j*k + c of step i >= 1 is child c of frontier slot j,
// drawn from row 1 + (i-1)*k + j.
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
  __shared__ int s_fc[kMaxNodes], s_ns[kMaxNodes];
  __shared__ uint32_t s_bits[kMaxNodes][kMaxWords];

  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const float *tp = topk_p + static_cast<int64_t>(b) * M;
  const int *ti = topk_id + static_cast<int64_t>(b) * M;
  for (int e = tid; e < M; e += kTreeThreads) {
    s_tp[e] = tp[e];
    s_tok[e] = ti[e];
    s_row[e] = -1;
    s_tree[e] = 0;
  }
  const int L = prefix_len[b];
  const int root = root_token[b];
  __syncthreads();

  // With N - 1 <= 64 as well, wave 0 also keeps the best 64 keys of the
  // pool so far (every step's sorted keys merged in) and marks the final
  // N - 1 itself.
  const bool wave_final = k * k <= kWave && N - 1 <= kWave;
  if (k * k <= kWave) {
    // Every step's k*k candidates fit one wave: wave 0 runs the steps in
    // registers, each frontier the first k lanes of a wave sort of the
    // step's order keys (lanes past the candidates hold 0, below any key).
    if (tid < kWave) {
      const int x = tid;
      // step 0: the root's children
      unsigned long long key = 0;
      if (x < k) {
        key = order_key(s_tp[x], x);
        s_score[x] = s_tp[x];
        s_par[x] = -1;
        s_key[x] = key;
      }
      key = wave_sort_keys_desc(key);
      unsigned long long best = key;               // best 64 of the pool so far, largest first
      int fe = entry_of_key(key);                  // lanes j < k: frontier slot j
      float fs = x < k ? s_tp[fe] : 0.f;           // its score
      // steps 1 .. S-1: expand every frontier slot, keep the best k
      for (int i = 1; i < S; ++i) {
        const int base = k + (i - 1) * k * k;
        const int f = __shfl(fe, x / k, kWave);
        const float fsc = __shfl(fs, x / k, kWave);
        if (x < k) s_row[fe] = 1 + (i - 1) * k + x;
        key = 0;
        if (x < k * k) {
          const int e = base + x;
          const float sc = fsc * s_tp[e];
          s_score[e] = sc;
          s_par[e] = f;
          key = order_key(sc, e);
          s_key[e] = key;
        }
        key = wave_sort_keys_desc(key);
        if (wave_final) best = wave_merge_top(best, key);
        fe = entry_of_key(key);
        fs = x < k ? s_score[fe] : 0.f;            // written by this wave above (LDS keeps a wave's order)
      }
      if (wave_final && x < N - 1) s_tree[entry_of_key(best)] = 1;   // keys are distinct: the top N-1 entries
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

  // final selection: the best N-1 pool entries, numbered in pool order
  if (!wave_final) {
    rank_block(s_key, 0, M, [&](int e, int r) { s_tree[e] = r < N - 1 ? 1 : 0; });
    __syncthreads();
  }
  const int per = (M + kTreeThreads - 1) / kTreeThreads;
  const int e0 = tid * per;
  int cnt = 0;
  for (int e = e0; e < min(M, e0 + per); ++e) cnt += s_tree[e];
  int t = 1 + block_exclusive_scan(cnt);   // tree index of this thread's first selected entry
  for (int e = e0; e < min(M, e0 + per); ++e) s_tree[e] = s_tree[e] ? t++ : -1;
  __syncthreads();

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

  // first child and next sibling: the smallest larger index with the node
  // as parent / with the same parent, found over all (n, m) pairs
  for (int n = tid; n < N; n += kTreeThreads) {
    s_fc[n] = INT_MAX;
    s_ns[n] = INT_MAX;
  }
  __syncthreads();
  for (int x = tid; x < N * N; x += kTreeThreads) {
    const int n = x / N, m = x % N;
    if (m <= n) continue;
    const int pm = s_tpar[m];
    if (pm == n) atomicMin(&s_fc[n], m);
    const int p = s_tpar[n];
    if (p >= 0 && pm == p) atomicMin(&s_ns[n], m);
  }
  const int W = (N + 31) / 32;
  for (int n = tid; n < N; n += kTreeThreads) {
    uint32_t bits[kMaxWords];
#pragma unroll
    for (int w = 0; w < kMaxWords; ++w) bits[w] = 0;
    int j = n;
    for (int hop = 0; hop <= S && j >= 0; ++hop) {
#pragma unroll
      for (int w = 0; w < kMaxWords; ++w)
        if (w == j / 32) bits[w] |= 1u << (j % 32);
      j = s_tpar[j];
    }
#pragma unroll
    for (int w = 0; w < kMaxWords; ++w) {
      s_bits[n][w] = bits[w];
      if (o_bits && w < W) o_bits[(ob + n) * W + w] = bits[w];
    }
    o_retrieve[ob + n] = static_cast<int>(ob + n);
  }
  __syncthreads();
  for (int n = tid; n < N; n += kTreeThreads) {
    o_next_token[ob + n] = s_fc[n] == INT_MAX ? -1 : s_fc[n];
    o_next_sibling[ob + n] = s_ns[n] == INT_MAX ? -1 : s_ns[n];
  }
  if (o_mask) {
    for (int x = tid; x < N * N; x += kTreeThreads) {
      const int r = x / N, c = x % N;
      o_mask[ob * N + x] = static_cast<uint8_t>((s_bits[r][c / 32] >> (c % 32)) & 1u);
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
  hipLaunchKernelGGL(build_tree_kernel, dim3(sh.B), dim3(kTreeThreads), lds, as_stream(stream), sh.k,
                     sh.S, sh.N, topk_p, topk_id, root_token, prefix_len, tokens, parent, depth,
                     positions, score, q_row, mask, mask_bits, retrieve_index, retrieve_next_token,
                     retrieve_next_sibling);
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
