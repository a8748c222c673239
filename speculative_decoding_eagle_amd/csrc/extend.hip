// Index preparation of the draft extend that follows a verify step ("EAGLE
// speculative decoding in four parts", "Self-test" answer 1: the draft model
// runs one extend over the accepted tokens to ready the next round;
// zero-to-sglang ch.10 section 3.1: draft, verify, then the draft-side
// extend; sglang PR #22883 "Modifications": under TLI the accepted target
// ids are mapped to draft ids for that extend).
//
// One 1024-thread workgroup: thread t owns requests t, t + 1024, ...; an
// exclusive scan of the commit lengths over the batch (chunks of 1024 with a
// carried total) gives each request's first row, and each thread then fills
// its own requests' rows (at most S + 1 each).  Launch-bound: a few kB move.
#include "common.hpp"

namespace sdv {
namespace {

constexpr int kExtThreads = 1024;

__device__ __forceinline__ int wave_inclusive_sum(int v) {
  const int lane = lane_id();
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int o = __shfl_up(v, off, kWave);
    if (lane >= off) v += o;
  }
  return v;
}

__global__ void __launch_bounds__(kExtThreads)
extend_prep_kernel(int B, int N, int S1, const int32_t *__restrict__ prefix_len,
                   const int32_t *__restrict__ commit_len, const int32_t *__restrict__ commit_tokens,
                   const int32_t *__restrict__ accept_path, const int32_t *__restrict__ t2d, int Vt,
                   int32_t *__restrict__ extend_start, int32_t *__restrict__ input_ids,
                   int32_t *__restrict__ positions, int32_t *__restrict__ hidden_index,
                   int32_t *__restrict__ last_index, int32_t *__restrict__ seq_len) {
  constexpr int NW = kExtThreads / kWave;
  __shared__ int s_wave[NW];
  __shared__ int s_carry;
  const int tid = threadIdx.x;
  const int w = tid / kWave;
  if (tid == 0) s_carry = 0;
  __syncthreads();
  // 1. exclusive scan of the (clamped) commit lengths
  for (int c0 = 0; c0 < B; c0 += kExtThreads) {
    const int b = c0 + tid;
    int c = b < B ? commit_len[b] : 0;
    c = c < 0 ? 0 : (c > S1 ? S1 : c);
    const int inc = wave_inclusive_sum(c);
    if (lane_id() == kWave - 1) s_wave[w] = inc;
    __syncthreads();
    int before = s_carry;
    for (int x = 0; x < w; ++x) before += s_wave[x];
    if (b < B) extend_start[b] = before + inc - c;
    __syncthreads();
    if (tid == kExtThreads - 1) s_carry = before + inc;
    __syncthreads();
  }
  if (tid == 0) extend_start[B] = s_carry;
  // 2. each thread fills the rows of the requests it scanned (its own
  //    extend_start writes, read back in program order)
  for (int b = tid; b < B; b += kExtThreads) {
    int c = commit_len[b];
    c = c < 0 ? 0 : (c > S1 ? S1 : c);
    const int start = extend_start[b];
    const int L = prefix_len[b];
    const int32_t *tok = commit_tokens + static_cast<int64_t>(b) * S1;
    const int32_t *path = accept_path + static_cast<int64_t>(b) * S1;
    for (int j = 0; j < c; ++j) {
      const int t = tok[j];
      const int u = path[j];
      int id = t;
      if (t2d) id = (t >= 0 && t < Vt) ? t2d[t] : -1;
      input_ids[start + j] = t < 0 ? -1 : id;
      positions[start + j] = L + 1 + j;
      hidden_index[start + j] = (u >= 0 && u < N) ? b * N + u : -1;
    }
    last_index[b] = c > 0 ? start + c - 1 : -1;
    seq_len[b] = L + 1 + c;
  }
}

}  // namespace
}  // namespace sdv

using namespace sdv;

extern "C" int32_t sdv_draft_extend_prep(int32_t B, int32_t N, int32_t S, const int32_t *prefix_len,
                                         const int32_t *commit_len, const int32_t *commit_tokens,
                                         const int32_t *accept_path, const int32_t *t2d, int32_t V_target,
                                         int32_t *extend_start, int32_t *input_ids, int32_t *positions,
                                         int32_t *hidden_index, int32_t *last_index, int32_t *seq_len,
                                         void *stream) {
  clear_error();
  SDV_REQUIRE(B >= 0 && N >= 1 && S >= 0, SDV_E_SHAPE, "draft_extend_prep: need B >= 0, N >= 1, S >= 0");
  SDV_REQUIRE(static_cast<int64_t>(B) * N < (1LL << 31) && static_cast<int64_t>(B) * (S + 1) < (1LL << 31),
              SDV_E_UNSUPPORTED, "draft_extend_prep: B * N and B * (S + 1) must fit in int32");
  SDV_REQUIRE(!t2d || V_target >= 1, SDV_E_SHAPE, "draft_extend_prep: a map needs V_target >= 1");
  SDV_REQUIRE(extend_start, SDV_E_NULL, "draft_extend_prep: NULL extend_start");
  if (B > 0) {
    SDV_REQUIRE(prefix_len && commit_len && commit_tokens && accept_path && input_ids && positions &&
                    hidden_index && last_index && seq_len,
                SDV_E_NULL, "draft_extend_prep: NULL pointer");
  }
  hipLaunchKernelGGL(extend_prep_kernel, dim3(1), dim3(kExtThreads), 0, as_stream(stream), B, N, S + 1,
                     prefix_len, commit_len, commit_tokens, accept_path, t2d, V_target, extend_start, input_ids,
                     positions, hidden_index, last_index, seq_len);
  return check_launch("extend_prep_kernel");
}
