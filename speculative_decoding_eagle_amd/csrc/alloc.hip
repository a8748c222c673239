// KV slot / page allocation around a speculative step ("EAGLE speculative
// decoding in four parts", "Drafting, verification and slots": page size 1
// reserves batch x topk x steps slots at once with the allocator's state
// backed up and rolled back after the step; page size > 1 extends each
// request with topk = 1 and duplicates the last partial page per branch
// with topk > 1; "Design trade-offs": allocate first, roll back after).
//
// The allocator lives in device memory: a stack of free unit ids
// (free_ids[0 .. top), the top one handed out first) and a state word array
// {top, pushes, error, 0}.  Every operation is one small kernel on the
// caller's stream, so a step allocates, rolls back and releases without a
// host round trip.  The allocating kernels run in one 1024-thread workgroup:
// a pass over the batch computes each request's need and checks its table
// row, a scan gives each request its place in the pop order, and only if the
// whole batch fits are ids popped (all or nothing).  The partial-page copies
// of the branch layout are a separate, bandwidth-bound kernel.
#include "common.hpp"

namespace sdv {
namespace {

constexpr int kAllocThreads = 1024;
constexpr int kAllocMaxBatch = 8192;          // requests per allocating call (LDS offsets)
constexpr int kCopyThreads = 256;

enum : int { kTop = 0, kPushes = 1, kError = 2 };
enum : int { kErrNoRoom = 1, kErrRestore = 2, kErrOverflow = 4, kErrState = 8, kErrSlot = 16 };

__device__ __forceinline__ void raise_error(int *state, int bits) { atomicOr(state + kError, bits); }

__global__ void alloc_init_kernel(int capacity, int *__restrict__ free_ids, int *__restrict__ state) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < capacity) free_ids[i] = capacity - 1 - i;
  if (i == 0) {
    state[kTop] = capacity;
    state[kPushes] = 0;
    state[kError] = 0;
    state[3] = 0;
  }
}

__global__ void alloc_backup_kernel(const int *__restrict__ state, int *__restrict__ backup) {
  backup[0] = state[kTop];
  backup[1] = state[kPushes];
}

__global__ void alloc_restore_kernel(int capacity, int *__restrict__ state, const int *__restrict__ backup) {
  const int top = backup[0];
  if (backup[1] != state[kPushes] || top < state[kTop] || top > capacity) {
    raise_error(state, kErrRestore);
    return;
  }
  state[kTop] = top;
}

__global__ void __launch_bounds__(kAllocThreads)
alloc_free_kernel(int capacity, int max_ids, int *__restrict__ free_ids, int *__restrict__ state,
                  const int *__restrict__ ids, const int *__restrict__ num_ids) {
  const int top = state[kTop];
  const int n = *num_ids;
  if (n < 0 || n > max_ids || top < 0 || top > capacity || top + n > capacity) {
    if (threadIdx.x == 0) raise_error(state, kErrOverflow);
    return;
  }
  for (int i = threadIdx.x; i < n; i += kAllocThreads) free_ids[top + i] = ids[i];
  __syncthreads();                      // every thread has read the old top
  if (threadIdx.x == 0) {
    state[kTop] = top + n;
    state[kPushes] += 1;
  }
}

__device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Exclusive scan of need(b) over b < B into s_off (LDS), plus the total; the
// block-wide flag s_bad collects any request whose check fails.  All threads
// return the total.
template <typename NeedFn>
__device__ int scan_needs(int B, NeedFn need, int *s_off, int *s_wave, int *s_carry) {
  const int tid = threadIdx.x;
  const int w = tid / kWave;
  if (tid == 0) *s_carry = 0;
  __syncthreads();
  for (int c0 = 0; c0 < B; c0 += kAllocThreads) {
    const int b = c0 + tid;
    const int v = b < B ? need(b) : 0;
    int inc = v;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int o = __shfl_up(inc, off, kWave);
      if (lane_id() >= off) inc += o;
    }
    if (lane_id() == kWave - 1) s_wave[w] = inc;
    __syncthreads();
    int before = *s_carry;
    for (int x = 0; x < w; ++x) before += s_wave[x];
    if (b < B) s_off[b] = before + inc - v;
    __syncthreads();
    if (tid == kAllocThreads - 1) *s_carry = before + inc;
    __syncthreads();
  }
  return *s_carry;
}

// Positions L .. L+n-1 of each request's own chain (L = seq_len[b]).
__global__ void __launch_bounds__(kAllocThreads)
alloc_extend_kernel(int capacity, int B, int P, int n, int max_pages, const int *__restrict__ free_ids,
                    int *__restrict__ state, int *__restrict__ table, const int *__restrict__ seq_len,
                    int *__restrict__ out_loc) {
  __shared__ int s_off[kAllocMaxBatch];
  __shared__ int s_wave[kAllocThreads / kWave];
  __shared__ int s_carry, s_bad;
  const int tid = threadIdx.x;
  if (tid == 0) s_bad = 0;
  __syncthreads();
  auto need = [&](int b) {
    const int L = seq_len[b];
    const int end = ceil_div(L + n, P);          // table entries the row must hold
    if (L < 0 || end > max_pages) atomicOr(&s_bad, 1);
    return P == 1 ? n : end - ceil_div(L, P);
  };
  const int total = scan_needs(B, need, s_off, s_wave, &s_carry);
  const int top = state[kTop];
  const bool ok = s_bad == 0 && top >= 0 && top <= capacity && total <= top;
  if (!ok) {
    for (int x = tid; x < B * n; x += kAllocThreads) out_loc[x] = -1;
    if (tid == 0) raise_error(state, (top < 0 || top > capacity) ? kErrState : kErrNoRoom);
    return;
  }
  // pop: request b takes stack entries top-1-s_off[b] downwards
  for (int b = tid; b < B; b += kAllocThreads) {
    const int L = seq_len[b];
    int *row = table + static_cast<int64_t>(b) * max_pages;
    const int first = P == 1 ? L : ceil_div(L, P);
    const int cnt = P == 1 ? n : ceil_div(L + n, P) - first;
    for (int t = 0; t < cnt; ++t) row[first + t] = free_ids[top - 1 - (s_off[b] + t)];
  }
  __syncthreads();                      // the new table entries are visible to the workgroup
  for (int x = tid; x < B * n; x += kAllocThreads) {
    const int b = x / n;
    const int pos = seq_len[b] + x % n;
    out_loc[x] = table[static_cast<int64_t>(b) * max_pages + pos / P] * P + pos % P;
  }
  if (tid == 0) state[kTop] = top - total;
}

// Per-branch regions: branch j of request b takes ceil((r + S) / P) pages,
// r = seq_len[b] mod P; its first r slots will hold the partial page's copy.
__global__ void __launch_bounds__(kAllocThreads)
alloc_branches_kernel(int capacity, int B, int P, int topk, int S, int maxpb, const int *__restrict__ free_ids,
                      int *__restrict__ state, const int *__restrict__ seq_len, int *__restrict__ branch_pages,
                      int *__restrict__ out_loc) {
  __shared__ int s_off[kAllocMaxBatch];
  __shared__ int s_wave[kAllocThreads / kWave];
  __shared__ int s_carry, s_bad;
  const int tid = threadIdx.x;
  if (tid == 0) s_bad = 0;
  __syncthreads();
  auto per_branch = [&](int b) { return ceil_div(seq_len[b] % P + S, P); };
  auto need = [&](int b) {
    if (seq_len[b] < 0) atomicOr(&s_bad, 1);
    return topk * per_branch(b);
  };
  const int total = scan_needs(B, need, s_off, s_wave, &s_carry);
  const int top = state[kTop];
  const bool ok = s_bad == 0 && top >= 0 && top <= capacity && total <= top;
  const int64_t nb = static_cast<int64_t>(B) * topk;
  if (!ok) {
    for (int64_t x = tid; x < nb * maxpb; x += kAllocThreads) branch_pages[x] = -1;
    for (int64_t x = tid; x < nb * S; x += kAllocThreads) out_loc[x] = -1;
    if (tid == 0) raise_error(state, (top < 0 || top > capacity) ? kErrState : kErrNoRoom);
    return;
  }
  for (int64_t x = tid; x < nb * maxpb; x += kAllocThreads) {
    const int b = static_cast<int>(x / (static_cast<int64_t>(topk) * maxpb));
    const int j = static_cast<int>(x / maxpb % topk);
    const int t = static_cast<int>(x % maxpb);
    const int pb = per_branch(b);
    branch_pages[x] = t < pb ? free_ids[top - 1 - (s_off[b] + j * pb + t)] : -1;
  }
  for (int64_t x = tid; x < nb * S; x += kAllocThreads) {
    const int b = static_cast<int>(x / (static_cast<int64_t>(topk) * S));
    const int j = static_cast<int>(x / S % topk);
    const int i = static_cast<int>(x % S);
    const int pb = per_branch(b);
    const int q = seq_len[b] % P + i;
    out_loc[x] = free_ids[top - 1 - (s_off[b] + j * pb + q / P)] * P + q % P;
  }
  __syncthreads();                      // every thread has read the old top
  if (tid == 0) state[kTop] = top - total;
}

// Copies the r = seq_len mod P rows of each request's partial page into the
// first page of each of its branches; one block per (request, branch, layer,
// pool), 16 bytes per thread and step.
__global__ void __launch_bounds__(kCopyThreads)
partial_copy_kernel(PoolPtrs pools, int layers, int topk, int P, int maxpb, int max_pages, int64_t num_slots,
                    int row16, const int *__restrict__ table, const int *__restrict__ seq_len,
                    const int *__restrict__ branch_pages, int *__restrict__ state) {
  const int64_t blk = blockIdx.x;
  const int pool_v = static_cast<int>(blk & 1);
  const int layer = static_cast<int>((blk >> 1) % layers);
  const int64_t bj = (blk >> 1) / layers;
  const int b = static_cast<int>(bj / topk);
  const int L = seq_len[b];
  const int r = L % P;
  const int dst_page = branch_pages[bj * maxpb];
  if (r == 0 || dst_page < 0) return;
  const int src_page = (L / P) < max_pages ? table[static_cast<int64_t>(b) * max_pages + L / P] : -1;
  const int64_t src = static_cast<int64_t>(src_page) * P;
  const int64_t dst = static_cast<int64_t>(dst_page) * P;
  if (src_page < 0 || src + r > num_slots || dst + r > num_slots) {
    if (threadIdx.x == 0) raise_error(state, kErrSlot);
    return;
  }
  uint4 *pool = reinterpret_cast<uint4 *>(pool_v ? pools.v[layer] : pools.k[layer]);
  const int64_t n16 = static_cast<int64_t>(r) * row16;
  for (int64_t x = threadIdx.x; x < n16; x += kCopyThreads) pool[dst * row16 + x] = pool[src * row16 + x];
}

}  // namespace
}  // namespace sdv

using namespace sdv;

extern "C" int32_t sdv_kv_alloc_init(int32_t capacity, int32_t *free_ids, int32_t *state, void *stream) {
  clear_error();
  SDV_REQUIRE(capacity >= 0, SDV_E_SHAPE, "kv_alloc_init: capacity < 0");
  SDV_REQUIRE(state && (capacity == 0 || free_ids), SDV_E_NULL, "kv_alloc_init: NULL pointer");
  const int blocks = capacity > 0 ? (capacity + 255) / 256 : 1;
  hipLaunchKernelGGL(alloc_init_kernel, dim3(blocks), dim3(256), 0, as_stream(stream), capacity, free_ids, state);
  return check_launch("alloc_init_kernel");
}

extern "C" int32_t sdv_kv_alloc_backup(const int32_t *state, int32_t *backup, void *stream) {
  clear_error();
  SDV_REQUIRE(state && backup, SDV_E_NULL, "kv_alloc_backup: NULL pointer");
  hipLaunchKernelGGL(alloc_backup_kernel, dim3(1), dim3(1), 0, as_stream(stream), state, backup);
  return check_launch("alloc_backup_kernel");
}

extern "C" int32_t sdv_kv_alloc_restore(int32_t capacity, int32_t *state, const int32_t *backup, void *stream) {
  clear_error();
  SDV_REQUIRE(state && backup, SDV_E_NULL, "kv_alloc_restore: NULL pointer");
  hipLaunchKernelGGL(alloc_restore_kernel, dim3(1), dim3(1), 0, as_stream(stream), capacity, state, backup);
  return check_launch("alloc_restore_kernel");
}

extern "C" int32_t sdv_kv_alloc_free(int32_t capacity, int32_t *free_ids, int32_t *state, const int32_t *ids,
                                     const int32_t *num_ids, int32_t max_ids, void *stream) {
  clear_error();
  SDV_REQUIRE(capacity >= 0 && max_ids >= 0, SDV_E_SHAPE, "kv_alloc_free: negative size");
  SDV_REQUIRE(state && num_ids && (capacity == 0 || free_ids) && (max_ids == 0 || ids), SDV_E_NULL,
              "kv_alloc_free: NULL pointer");
  hipLaunchKernelGGL(alloc_free_kernel, dim3(1), dim3(kAllocThreads), 0, as_stream(stream), capacity, max_ids,
                     free_ids, state, ids, num_ids);
  return check_launch("alloc_free_kernel");
}

extern "C" int32_t sdv_kv_alloc_extend(int32_t capacity, int32_t *free_ids, int32_t *state, int32_t B,
                                       int32_t page, int32_t n, int32_t *page_table, int32_t max_pages,
                                       const int32_t *seq_len, int32_t *out_loc, void *stream) {
  clear_error();
  SDV_REQUIRE(capacity >= 0 && B >= 0 && page >= 1 && n >= 0 && max_pages >= 1, SDV_E_SHAPE,
              "kv_alloc_extend: need capacity, B, n >= 0, page >= 1, max_pages >= 1");
  SDV_REQUIRE(B <= kAllocMaxBatch, SDV_E_UNSUPPORTED, "kv_alloc_extend: B=%d above %d", B, kAllocMaxBatch);
  SDV_REQUIRE(static_cast<int64_t>(B) * n < (1LL << 31), SDV_E_UNSUPPORTED, "kv_alloc_extend: B*n too large");
  SDV_REQUIRE(state, SDV_E_NULL, "kv_alloc_extend: NULL state");
  if (B == 0) return SDV_OK;
  SDV_REQUIRE(free_ids && page_table && seq_len && (n == 0 || out_loc), SDV_E_NULL,
              "kv_alloc_extend: NULL pointer");
  hipLaunchKernelGGL(alloc_extend_kernel, dim3(1), dim3(kAllocThreads), 0, as_stream(stream), capacity, B, page, n,
                     max_pages, free_ids, state, page_table, seq_len, out_loc);
  return check_launch("alloc_extend_kernel");
}

extern "C" int32_t sdv_kv_alloc_branches(int32_t capacity, int32_t *free_ids, int32_t *state,
                                         sdv_branch_shape sh, uint16_t *const *k_pools,
                                         uint16_t *const *v_pools, const int32_t *page_table,
                                         const int32_t *seq_len, int32_t *branch_pages, int32_t *out_loc,
                                         void *stream) {
  clear_error();
  SDV_REQUIRE(capacity >= 0 && sh.B >= 0 && sh.page >= 1 && sh.topk >= 1 && sh.S >= 1 && sh.max_pages >= 1,
              SDV_E_SHAPE, "kv_alloc_branches: need B >= 0, page, topk, S, max_pages >= 1");
  SDV_REQUIRE(sh.B <= kAllocMaxBatch, SDV_E_UNSUPPORTED, "kv_alloc_branches: B=%d above %d", sh.B,
              kAllocMaxBatch);
  const int maxpb = sdv_kv_branch_pages(sh.page, sh.S);
  SDV_REQUIRE(static_cast<int64_t>(sh.B) * sh.topk * (maxpb + sh.S) < (1LL << 31), SDV_E_UNSUPPORTED,
              "kv_alloc_branches: batch too large");
  SDV_REQUIRE(state, SDV_E_NULL, "kv_alloc_branches: NULL state");
  if (sh.B == 0) return SDV_OK;
  SDV_REQUIRE(free_ids && page_table && seq_len && branch_pages && out_loc, SDV_E_NULL,
              "kv_alloc_branches: NULL pointer");
  PoolPtrs pp;
  const bool copy = sh.page > 1 && sh.layers > 0;
  if (copy) {
    SDV_REQUIRE(sh.layers <= kMaxLayers, SDV_E_UNSUPPORTED, "kv_alloc_branches: layers=%d above %d", sh.layers,
                kMaxLayers);
    SDV_REQUIRE(sh.Hkv >= 1 && sh.D >= 1 && (static_cast<int64_t>(sh.Hkv) * sh.D) % 8 == 0, SDV_E_UNSUPPORTED,
                "kv_alloc_branches: Hkv*D must be a multiple of 8");
    SDV_REQUIRE(k_pools && v_pools, SDV_E_NULL, "kv_alloc_branches: NULL pool array");
    for (int l = 0; l < sh.layers; ++l) {
      SDV_REQUIRE(k_pools[l] && v_pools[l], SDV_E_NULL, "kv_alloc_branches: NULL pool of layer %d", l);
      SDV_REQUIRE(reinterpret_cast<uintptr_t>(k_pools[l]) % 16 == 0 &&
                      reinterpret_cast<uintptr_t>(v_pools[l]) % 16 == 0,
                  SDV_E_SHAPE, "kv_alloc_branches: pools must be 16-byte aligned");
      pp.k[l] = k_pools[l];
      pp.v[l] = v_pools[l];
    }
    for (int l = sh.layers; l < kMaxLayers; ++l) pp.k[l] = pp.v[l] = nullptr;
  }
  hipStream_t st = as_stream(stream);
  hipLaunchKernelGGL(alloc_branches_kernel, dim3(1), dim3(kAllocThreads), 0, st, capacity, sh.B, sh.page, sh.topk,
                     sh.S, maxpb, free_ids, state, seq_len, branch_pages, out_loc);
  int32_t rc = check_launch("alloc_branches_kernel");
  if (rc != SDV_OK || !copy) return rc;
  const int64_t blocks = static_cast<int64_t>(sh.B) * sh.topk * sh.layers * 2;
  SDV_REQUIRE(blocks < (1LL << 31), SDV_E_UNSUPPORTED, "kv_alloc_branches: too many copies");
  const int row16 = static_cast<int>(static_cast<int64_t>(sh.Hkv) * sh.D / 8);
  hipLaunchKernelGGL(partial_copy_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kCopyThreads), 0, st, pp,
                     sh.layers, sh.topk, sh.page, maxpb, sh.max_pages, sh.num_slots, row16, page_table, seq_len,
                     branch_pages, state);
  return check_launch("partial_copy_kernel");
}

extern "C" int32_t sdv_kv_branch_pages(int32_t page, int32_t S) {
  if (page < 1 || S < 1) return 0;
  return page == 1 ? S : (page - 1 + S + page - 1) / page;
}
