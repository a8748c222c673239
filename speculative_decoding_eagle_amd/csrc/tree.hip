// A2-A4: candidate tree from the per-step top-k ("[SGLang] Multi-Layer
// EAGLE" section 2, select_top_k_tokens / tree_info; build_eagle_tree in
// "EAGLE speculative decoding in four parts", "Drafting, verification and
// slots"), plus positions, the tree mask and the retrieve arrays
// (zero-to-sglang ch.10 section 5.2).
//
// Latency-bound integer work: one 256-thread block per request keeps the
// whole candidate pool in LDS.  Every selection (each step's frontier and the
// final best N-1) is a rank computation under the strict order
// (score desc, pool index asc): an entry's rank is the number of entries that
// beat it, so ranks are unique and the result is deterministic.
#include "common.hpp"

namespace sdv {
namespace {

constexpr int kTreeThreads = 256;
constexpr int kMaxPool = 2048;
constexpr int kMaxNodes = 256;
constexpr int kMaxWords = kMaxNodes / 32;

__device__ __forceinline__ bool beats(const float *sc, int a, int b) {
  return sc[a] > sc[b] || (sc[a] == sc[b] && a < b);
}

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
  const int R = 1 + (S - 1) * k;
  float *s_score = reinterpret_cast<float *>(smem);
  int *s_token = reinterpret_cast<int *>(s_score + M);
  int *s_par = s_token + M;      // pool index of the parent, -1 = root
  int *s_step = s_par + M;
  int *s_row = s_step + M;       // draft row of the entry's children, -1
  int *s_tree = s_row + M;       // tree index, -1 if not selected
  __shared__ int s_front[32];
  __shared__ int s_tpar[kMaxNodes];
  __shared__ uint32_t s_bits[kMaxNodes][kMaxWords];
  __shared__ int s_scan[kTreeThreads];

  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const float *tp = topk_p + static_cast<int64_t>(b) * R * k;
  const int *ti = topk_id + static_cast<int64_t>(b) * R * k;

  // step 0: the root's children, in rank order they already form the frontier
  for (int c = tid; c < k; c += kTreeThreads) {
    s_score[c] = tp[c];
    s_token[c] = ti[c];
    s_par[c] = -1;
    s_step[c] = 0;
    s_row[c] = -1;
    s_tree[c] = -1;
  }
  __syncthreads();
  for (int c = tid; c < k; c += kTreeThreads) {
    int r = 0;
    for (int o = 0; o < k; ++o) r += beats(s_score, o, c);
    s_front[r] = c;
  }
  __syncthreads();

  // steps 1 .. S-1: expand every frontier slot, keep the best k as the next frontier
  for (int i = 1; i < S; ++i) {
    const int base = k + (i - 1) * k * k;
    for (int x = tid; x < k * k; x += kTreeThreads) {
      const int j = x / k, c = x % k;
      const int f = s_front[j];
      const int row = 1 + (i - 1) * k + j;
      const int e = base + x;
      s_score[e] = s_score[f] * tp[row * k + c];
      s_token[e] = ti[row * k + c];
      s_par[e] = f;
      s_step[e] = i;
      s_row[e] = -1;
      s_tree[e] = -1;
    }
    for (int j = tid; j < k; j += kTreeThreads) s_row[s_front[j]] = 1 + (i - 1) * k + j;
    __syncthreads();
    for (int x = tid; x < k * k; x += kTreeThreads) {
      const int e = base + x;
      int r = 0;
      for (int o = base; o < base + k * k; ++o) r += beats(s_score, o, e);
      if (r < k) s_front[r] = e;
    }
    __syncthreads();
  }

  // final selection: the best N-1 pool entries
  const int per = (M + kTreeThreads - 1) / kTreeThreads;
  const int e0 = tid * per;
  int cnt = 0;
  for (int e = e0; e < min(M, e0 + per); ++e) {
    int r = 0;
    for (int o = 0; o < M; ++o) r += beats(s_score, o, e);
    const bool sel = r < N - 1;
    s_tree[e] = sel ? 1 : 0;
    cnt += sel;
  }
  s_scan[tid] = cnt;
  __syncthreads();
  // inclusive Hillis-Steele scan of the per-thread counts
  for (int off = 1; off < kTreeThreads; off <<= 1) {
    const int add = tid >= off ? s_scan[tid - off] : 0;
    __syncthreads();
    s_scan[tid] += add;
    __syncthreads();
  }
  int t = 1 + s_scan[tid] - cnt;   // tree index of this thread's first selected entry
  for (int e = e0; e < min(M, e0 + per); ++e) {
    if (s_tree[e]) {
      s_tree[e] = t++;
    } else {
      s_tree[e] = -1;
    }
  }
  __syncthreads();

  const int64_t ob = static_cast<int64_t>(b) * N;
  const int L = prefix_len[b];
  if (tid == 0) {
    o_tokens[ob] = root_token[b];
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
    o_tokens[ob + te] = s_token[e];
    o_parent[ob + te] = tpar;
    o_depth[ob + te] = s_step[e] + 1;
    o_positions[ob + te] = L + s_step[e] + 1;
    o_score[ob + te] = s_score[e];
    o_qrow[ob + te] = s_row[e];
    s_tpar[te] = tpar;
  }
  __syncthreads();

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
    int nt = -1, ns = -1;
    const int p = s_tpar[n];
    for (int m = n + 1; m < N; ++m) {
      const int pm = s_tpar[m];
      if (nt < 0 && pm == n) nt = m;
      if (ns < 0 && p >= 0 && pm == p) ns = m;
    }
    o_next_token[ob + n] = nt;
    o_next_sibling[ob + n] = ns;
    o_retrieve[ob + n] = static_cast<int>(ob + n);
  }
  if (o_mask) {
    __syncthreads();
    for (int x = tid; x < N * N; x += kTreeThreads) {
      const int r = x / N, c = x % N;
      o_mask[ob * N + x] = static_cast<uint8_t>((s_bits[r][c / 32] >> (c % 32)) & 1u);
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
  const size_t lds = static_cast<size_t>(M) * 6 * sizeof(int);
  hipLaunchKernelGGL(build_tree_kernel, dim3(sh.B), dim3(kTreeThreads), lds, as_stream(stream), sh.k,
                     sh.S, sh.N, topk_p, topk_id, root_token, prefix_len, tokens, parent, depth,
                     positions, score, q_row, mask, mask_bits, retrieve_index, retrieve_next_token,
                     retrieve_next_sibling);
  return check_launch("build_tree_kernel");
}
