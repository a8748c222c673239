// A8: keep the accepted path's KV and release the rest of the tree's
// allocation ("EAGLE speculative decoding in four parts", "Self-test"
// answer 3 and "Drafting, verification and slots"; zero-to-sglang ch.10
// section 5.2).
//
// page == 1: an index remap of the slot map (one block per request), no KV
// bytes move.  page > 1: a per-request kernel reads the moved tokens' source
// and destination slots once (into the workspace) and then clears and lists
// the released tail pages; a second kernel copies the moved K/V rows
// (16-byte vectors, one block per request x layer x pool, one dependent load
// before its copies).  The freed lists of all requests are laid out in batch
// order; each block finds its offset from the accept lengths of the requests
// before it.
#include "common.hpp"

namespace sdv {
namespace {

constexpr int kCmpThreads = 256;
constexpr int kCopyBatch = 4;     // 16-byte vectors per thread per batch

__device__ __forceinline__ int clamp_accept(int a, int S, int N) {
  const int hi = min(S, N - 1);
  return a < 0 ? 0 : (a > hi ? hi : a);
}

// Released ids of request r.
__device__ __forceinline__ int released(int r, const int *prefix_len, const int *accept_len, int S, int N,
                                        int page) {
  const int a = clamp_accept(accept_len[r], S, N);
  if (page == 1) return N - 1 - a;
  const int L = prefix_len[r];
  const int first_free = (L + a + 1 + page - 1) / page;
  const int last_used = (L + N - 1) / page;
  return last_used >= first_free ? last_used - first_free + 1 : 0;
}

// Sum of released(r) over r < upto (all threads get it): per-thread sums,
// a wave sum, then the four waves' sums in order.
__device__ int released_before(int upto, const int *prefix_len, const int *accept_len, int S, int N,
                               int page) {
  constexpr int kWaves = kCmpThreads / kWave;
  __shared__ int s_part[kWaves];
  int acc = 0;
  for (int r = threadIdx.x; r < upto; r += kCmpThreads) acc += released(r, prefix_len, accept_len, S, N, page);
#pragma unroll
  for (int off = kWave / 2; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, kWave);
  if (lane_id() == 0) s_part[threadIdx.x / kWave] = acc;
  __syncthreads();
  int tot = 0;
#pragma unroll
  for (int j = 0; j < kWaves; ++j) tot += s_part[j];
  __syncthreads();
  return tot;
}

__global__ void __launch_bounds__(kCmpThreads)
remap_slots_kernel(int B, int N, int S, int max_pages, int *__restrict__ table,
                   const int *__restrict__ prefix_len, const int *__restrict__ accept_len,
                   const int *__restrict__ accept_path, int *__restrict__ new_len, int *__restrict__ freed,
                   int *__restrict__ num_freed) {
  __shared__ int s_old[256];
  __shared__ int s_kept[256];
  __shared__ int s_scan[kCmpThreads / kWave];
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int L = prefix_len[b];
  const int a = clamp_accept(accept_len[b], S, N);
  int *row = table + static_cast<int64_t>(b) * max_pages;
  const bool ok = L >= 0 && L + N <= max_pages;
  const int base = released_before(b, prefix_len, accept_len, S, N, 1);
  if (b == 0) {
    const int tot = released_before(B, prefix_len, accept_len, S, N, 1);
    if (tid == 0) *num_freed = tot;
  }
  if (tid < N) {
    s_old[tid] = ok ? row[L + tid] : -1;
    s_kept[tid] = 0;
  }
  __syncthreads();
  if (tid <= a) {
    int pj = accept_path[static_cast<int64_t>(b) * (S + 1) + tid];
    pj = pj < 0 ? 0 : (pj >= N ? N - 1 : pj);
    s_kept[pj] = 1;
  }
  __syncthreads();
  // exclusive scan of the not-kept flags gives each released slot its
  // place: a ballot per wave, then the waves before this one
  const bool flag = tid < N && !s_kept[tid];
  const unsigned long long m = __ballot(flag);
  if (lane_id() == 0) s_scan[tid / kWave] = __popcll(m);
  __syncthreads();
  int before = __popcll(m & ((1ull << lane_id()) - 1ull));
  for (int w = 0; w < tid / kWave; ++w) before += s_scan[w];
  if (flag) freed[base + before] = s_old[tid];
  if (ok && tid < N) {
    int v = -1;
    if (tid <= a) {
      int pj = accept_path[static_cast<int64_t>(b) * (S + 1) + tid];
      pj = pj < 0 ? 0 : (pj >= N ? N - 1 : pj);
      v = s_old[pj];
    }
    row[L + tid] = v;
  }
  if (tid == 0) new_len[b] = L + a + 1;
}

// page > 1, first kernel (one block per request): the source and
// destination slots of every moved token (path[d] != d, d = 1..a) go to the
// workspace as pairs, then the released tail pages are cleared and listed.
// The table is read and written here only, so reading the moved tokens'
// slots before the release needs no ordering across blocks.
__global__ void __launch_bounds__(kCmpThreads)
prep_pages_kernel(int B, int N, int S, int page, int max_pages, int64_t num_slots, int *__restrict__ table,
                  const int *__restrict__ prefix_len, const int *__restrict__ accept_len,
                  const int *__restrict__ accept_path, int2 *__restrict__ pairs, int *__restrict__ counts,
                  int *__restrict__ new_len, int *__restrict__ freed, int *__restrict__ num_freed) {
  __shared__ int s_count;
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int L = prefix_len[b];
  const int a = clamp_accept(accept_len[b], S, N);
  const bool ok = L >= 0 && static_cast<int64_t>(L) + N <= static_cast<int64_t>(max_pages) * page;
  int *row = table + static_cast<int64_t>(b) * max_pages;
  const int *path = accept_path + static_cast<int64_t>(b) * (S + 1);
  if (tid == 0) s_count = 0;
  const int base = released_before(b, prefix_len, accept_len, S, N, page);   // (has barriers)
  if (b == 0) {
    const int tot = released_before(B, prefix_len, accept_len, S, N, page);
    if (tid == 0) *num_freed = tot;
  }
  // moved tokens: thread d - 1 takes row d (d = 1..a, at most 63 of them,
  // one wave); the kept ones are packed in increasing d by a ballot
  if (tid < kWave) {
    const int d = tid + 1;
    bool mv = false;
    int2 pr = make_int2(0, 0);
    if (ok && d <= a) {
      int pd = path[d];
      pd = pd < 0 ? 0 : (pd >= N ? N - 1 : pd);
      const int ps = L + pd, pdst = L + d;
      const int64_t ss = static_cast<int64_t>(row[ps / page]) * page + ps % page;
      const int64_t sd = static_cast<int64_t>(row[pdst / page]) * page + pdst % page;
      mv = pd != d && ss >= 0 && ss < num_slots && sd >= 0 && sd < num_slots;
      pr = make_int2(static_cast<int>(ss), static_cast<int>(sd));
    }
    const unsigned long long m = __ballot(mv);
    const int slot = __popcll(m & ((1ull << tid) - 1ull));
    if (mv) pairs[static_cast<int64_t>(b) * S + slot] = pr;
    if (tid == 0) s_count = __popcll(m);
  }
  __syncthreads();                       // the moved tokens' slots are read before the release below
  if (tid == 0) counts[b] = s_count;
  const int first_free = (L + a + 1 + page - 1) / page;
  const int last_used = (L + N - 1) / page;
  for (int pg = first_free + tid; pg <= last_used; pg += kCmpThreads) {
    const bool in = pg >= 0 && pg < max_pages;
    freed[base + pg - first_free] = in ? row[pg] : -1;
    if (in) row[pg] = -1;
  }
  if (tid == 0) new_len[b] = L + a + 1;
}

// page > 1, second kernel: one block per (request, group of kLayerGroup
// layers) copies the request's moved K and V rows [Hkv, D] of those layers,
// 16-byte vectors.  The count and the pairs load together (pairs past the
// count are not used); then every read of the block is in flight before its
// first write, which also makes the copy safe where a row's source is a
// lower row's destination (the path is increasing and path[d] >= d).
constexpr int kLayerGroup = 4;
constexpr int kCopyPer = 16;              // 16-byte vectors per thread per pass

__global__ void __launch_bounds__(kCmpThreads)
copy_pairs_kernel(PoolPtrs pools, int layers, int S, int row16, const int2 *__restrict__ pairs,
                  const int *__restrict__ counts) {
  const int ngroups = (layers + kLayerGroup - 1) / kLayerGroup;
  const int b = blockIdx.x / ngroups;
  const int l0 = (blockIdx.x % ngroups) * kLayerGroup;
  const int nl = min(kLayerGroup, layers - l0);
  const int2 *pr = pairs + static_cast<int64_t>(b) * S;
  const int n = counts[b];
  // item x: pool p = x % 2, layer l0 + (x / 2) % nl, row (x / 2 / nl) / row16, chunk % row16
  const int items = n * row16 * nl * 2;
  for (int first = 0; first < items; first += kCopyPer * kCmpThreads) {
    uint4 buf[kCopyPer];
    uint4 *dst[kCopyPer];
#pragma unroll
    for (int j = 0; j < kCopyPer; ++j) {
      const int x = first + j * kCmpThreads + static_cast<int>(threadIdx.x);
      dst[j] = nullptr;
      if (x < items) {
        const int c16 = x % row16;
        const int y = x / row16;
        const int p = y & 1;
        const int ly = (y >> 1) % nl;
        const int r = (y >> 1) / nl;
        const int2 sd = pr[r];
        uint4 *pool = reinterpret_cast<uint4 *>(p ? pools.v[l0 + ly] : pools.k[l0 + ly]);
        buf[j] = pool[static_cast<int64_t>(sd.x) * row16 + c16];
        dst[j] = pool + static_cast<int64_t>(sd.y) * row16 + c16;
      }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kCopyPer; ++j)
      if (dst[j]) *dst[j] = buf[j];
    __syncthreads();
  }
}

}  // namespace
}  // namespace sdv

using namespace sdv;

// Workspace (page > 1): the moved tokens' (source, destination) slot pairs,
// S per request, then one count per request.
extern "C" size_t sdv_compact_kv_workspace_size(sdv_kv_shape sh) {
  if (sh.page <= 1 || sh.B <= 0 || sh.S < 0) return 0;
  Carver c(nullptr);
  c.take<int2>(static_cast<size_t>(sh.B) * (sh.S > 0 ? sh.S : 1));
  c.take<int>(static_cast<size_t>(sh.B));
  return c.bytes();
}

extern "C" int32_t sdv_compact_kv(sdv_kv_shape sh, uint16_t *const *k_pools, uint16_t *const *v_pools,
                                  int32_t *page_table, const int32_t *prefix_len,
                                  const int32_t *accept_len, const int32_t *accept_path,
                                  int32_t *new_len, int32_t *freed, int32_t *num_freed, void *ws,
                                  size_t ws_bytes, void *stream) {
  clear_error();
  SDV_REQUIRE(sh.B >= 0 && sh.N >= 1 && sh.S >= 0 && sh.page >= 1 && sh.max_pages >= 1, SDV_E_SHAPE,
              "compact_kv: need B >= 0, N >= 1, S >= 0, page >= 1, max_pages >= 1");
  SDV_REQUIRE(sh.N <= 256, SDV_E_UNSUPPORTED, "compact_kv: N=%d above 256", sh.N);
  if (sh.B == 0) return SDV_OK;
  SDV_REQUIRE(page_table && prefix_len && accept_len && accept_path && new_len && freed && num_freed,
              SDV_E_NULL, "compact_kv: NULL pointer");
  hipStream_t st = as_stream(stream);
  if (sh.page == 1) {
    hipLaunchKernelGGL(remap_slots_kernel, dim3(sh.B), dim3(kCmpThreads), 0, st, sh.B, sh.N, sh.S,
                       sh.max_pages, page_table, prefix_len, accept_len, accept_path, new_len, freed,
                       num_freed);
    return check_launch("remap_slots_kernel");
  }
  SDV_REQUIRE(sh.layers >= 1 && sh.layers <= kMaxLayers, SDV_E_UNSUPPORTED,
              "compact_kv: layers=%d outside [1, %d]", sh.layers, kMaxLayers);
  SDV_REQUIRE(sh.Hkv >= 1 && sh.D >= 1 && (static_cast<int64_t>(sh.Hkv) * sh.D) % 8 == 0, SDV_E_UNSUPPORTED,
              "compact_kv: Hkv*D must be a multiple of 8");
  SDV_REQUIRE(sh.S <= 63, SDV_E_UNSUPPORTED, "compact_kv: S=%d above 63 with page > 1", sh.S);
  SDV_REQUIRE(k_pools && v_pools, SDV_E_NULL, "compact_kv: NULL pool array");
  PoolPtrs pp;
  for (int l = 0; l < sh.layers; ++l) {
    SDV_REQUIRE(k_pools[l] && v_pools[l], SDV_E_NULL, "compact_kv: NULL pool of layer %d", l);
    SDV_REQUIRE(reinterpret_cast<uintptr_t>(k_pools[l]) % 16 == 0 &&
                    reinterpret_cast<uintptr_t>(v_pools[l]) % 16 == 0,
                SDV_E_SHAPE, "compact_kv: pools must be 16-byte aligned");
    pp.k[l] = k_pools[l];
    pp.v[l] = v_pools[l];
  }
  for (int l = sh.layers; l < kMaxLayers; ++l) pp.k[l] = pp.v[l] = nullptr;
  const int row16 = static_cast<int>(static_cast<int64_t>(sh.Hkv) * sh.D / 8);
  const size_t need = sdv_compact_kv_workspace_size(sh);
  SDV_REQUIRE(ws && ws_bytes >= need, SDV_E_WORKSPACE, "compact_kv: workspace of %zu bytes needed", need);
  Carver cv(ws);
  int2 *pairs = cv.take<int2>(static_cast<size_t>(sh.B) * (sh.S > 0 ? sh.S : 1));
  int *counts = cv.take<int>(static_cast<size_t>(sh.B));
  hipLaunchKernelGGL(prep_pages_kernel, dim3(sh.B), dim3(kCmpThreads), 0, st, sh.B, sh.N, sh.S, sh.page,
                     sh.max_pages, sh.num_slots, page_table, prefix_len, accept_len, accept_path, pairs, counts,
                     new_len, freed, num_freed);
  int32_t rc = check_launch("prep_pages_kernel");
  if (rc != SDV_OK) return rc;
  const int64_t blocks = static_cast<int64_t>(sh.B) * ((sh.layers + kLayerGroup - 1) / kLayerGroup);
  hipLaunchKernelGGL(copy_pairs_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kCmpThreads), 0, st, pp,
                     sh.layers, sh.S, row16, pairs, counts);
  return check_launch("copy_pairs_kernel");
}
