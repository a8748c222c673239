// A6-A7: target row reductions and the accept walk (zero-to-sglang ch.10
// sections 3.3, 4.1, 5.1; verify_tree_greedy and the other verification
// kernels in "EAGLE speculative decoding in four parts", "Drafting,
// verification and slots").
//
// The walk of one request is sequential in depth, but every row it reads is
// 4*V bytes, so a single wave per request cannot pull HBM bandwidth.  Each
// request is served by a group of W workgroups, each owning a contiguous
// slice of the vocabulary.  One cooperative launch keeps all groups
// resident; a group synchronises through a per-request arrival counter
// (agent-scope release/acquire) whenever the walk needs a row-wide value:
//   greedy     -- the argmax of the current node's target row;
//   stochastic -- each rejection's fixed-point residual mass, and the draw.
// Every workgroup of a group reduces the same W partials in the same order,
// so all of them take the same decisions without a second barrier.
// Partial slots form a ring of two: a workgroup only reaches barrier n+1
// after every workgroup has consumed barrier n-1's partials.
// Every spin is bounded; on timeout the kernel records an error flag and
// carries on, so every wave always exits.
#include <climits>
#include <cmath>

#include "common.hpp"

namespace sdv {
namespace {

constexpr int kAccThreads = 256;
constexpr int kAccWaves = kAccThreads / kWave;
constexpr int kMaxGroup = 64;          // workgroups per request
constexpr int kMaxLevels = 256;        // rejections at one node (children of one node)
constexpr unsigned kSpinLimit = 1u << 26;

struct AcceptArgs {
  int B, N, S, V, R, mode, eos;
  int W, chunk, b0;                    // group size, slice length, first request of this launch
  bool vec;
  const int *remaining;
  const int *tokens, *next_token, *next_sibling, *q_row;
  const float *target, *draft, *u_accept, *u_draw;
  int *accept_len, *accept_path, *commit_tokens, *commit_len, *next_root;
  unsigned *ctr;                       // [B] arrival counters (zeroed before the launch)
  unsigned long long *part;            // [B][2][kMaxGroup]
  unsigned *err;                       // [1] timeout flag
};

__device__ __forceinline__ unsigned long long pack_best(float v, int i) {
  return (static_cast<unsigned long long>(__float_as_uint(v)) << 32) | static_cast<unsigned>(i);
}
__device__ __forceinline__ float unpack_v(unsigned long long x) {
  return __uint_as_float(static_cast<unsigned>(x >> 32));
}
__device__ __forceinline__ int unpack_i(unsigned long long x) {
  return static_cast<int>(static_cast<unsigned>(x & 0xffffffffu));
}

__device__ __forceinline__ void store_part(unsigned long long *p, unsigned long long v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned long long load_part(unsigned long long *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Arrival barrier of the W workgroups serving one request.  `gen` counts the
// barriers this workgroup has passed; the n-th barrier completes at n*W.
__device__ void group_barrier(unsigned *ctr, unsigned &gen, int W, unsigned *err) {
  __syncthreads();
  ++gen;
  if (threadIdx.x == 0) {
    __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    const unsigned target = gen * static_cast<unsigned>(W);
    unsigned spins = 0;
    while (__hip_atomic_load(ctr, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) < target) {
      __builtin_amdgcn_s_sleep(1);
      if (++spins > kSpinLimit) {
        __hip_atomic_store(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
    }
  }
  __syncthreads();
}

// ------------------------------------------------------------ block reductions

__device__ void block_best(float &v, int &i) {
  __shared__ float sv[kAccWaves];
  __shared__ int si[kAccWaves];
  wave_best(v, i);
  const int w = threadIdx.x / kWave;
  if (lane_id() == 0) {
    sv[w] = v;
    si[w] = i;
  }
  __syncthreads();
  v = sv[0];
  i = si[0];
  for (int x = 1; x < kAccWaves; ++x)
    if (better(sv[x], si[x], v, i)) {
      v = sv[x];
      i = si[x];
    }
  __syncthreads();
}

__device__ unsigned long long block_sum(unsigned long long x) {
  __shared__ unsigned long long s[kAccWaves];
  x = wave_sum_u64(x);
  const int w = threadIdx.x / kWave;
  if (lane_id() == 0) s[w] = x;
  __syncthreads();
  unsigned long long t = 0;
  for (int j = 0; j < kAccWaves; ++j) t += s[j];
  __syncthreads();
  return t;
}

// Exclusive block scan of one u64 per thread; returns the exclusive prefix,
// `total` receives the block sum.
__device__ unsigned long long block_exclusive_scan(unsigned long long x, unsigned long long &total) {
  __shared__ unsigned long long s[kAccWaves];
  unsigned long long inc = x;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const unsigned long long y = __shfl_up(inc, off, kWave);
    if (lane_id() >= off) inc += y;
  }
  const int w = threadIdx.x / kWave;
  if (lane_id() == kWave - 1) s[w] = inc;
  __syncthreads();
  unsigned long long before = 0;
  total = 0;
  for (int j = 0; j < kAccWaves; ++j) {
    if (j < w) before += s[j];
    total += s[j];
  }
  __syncthreads();
  return before + inc - x;
}

// ------------------------------------------------------- sampling arithmetic

// t at one vocabulary entry after `lev` rejections at the current node:
// t <- fp32(double(max(t - q, 0)) / (double(S_j) * 2^-40)) for every level j
// whose residual mass S_j was non-zero.
__device__ __forceinline__ float t_at(float p, float q, const unsigned long long *Slev, int lev) {
  float t = p;
  for (int j = 0; j < lev; ++j) {
    const unsigned long long Sj = Slev[j];
    if (Sj == 0) continue;
    const float r = fmaxf(t - q, 0.0f);
    t = static_cast<float>(static_cast<double>(r) / (static_cast<double>(Sj) * 0x1p-40));
  }
  return t;
}

enum MassKind { kResidual = 0, kT = 1 };

__device__ __forceinline__ unsigned long long mass_of(float p, float q, const unsigned long long *Slev,
                                                      int lev, int kind) {
  const float t = t_at(p, q, Slev, lev);
  const float w = kind == kResidual ? fmaxf(t - q, 0.0f) : t;
  return static_cast<unsigned long long>(floor(static_cast<double>(w) * 0x1p40));
}

// ------------------------------------------------------------------- kernel

__global__ void __launch_bounds__(kAccThreads) accept_kernel(AcceptArgs a) {
  const int b = a.b0 + static_cast<int>(blockIdx.x) / a.W;
  const int c = static_cast<int>(blockIdx.x) % a.W;
  if (b >= a.B) return;
  const int tid = threadIdx.x;
  const int V = a.V;
  const int lo = min(V, c * a.chunk);
  const int hi = min(V, lo + a.chunk);
  unsigned *ctr = a.ctr + b;
  unsigned long long *ring = a.part + static_cast<int64_t>(b) * 2 * kMaxGroup;
  unsigned gen = 0;

  __shared__ int s_path[66];
  __shared__ int s_out[66];
  __shared__ unsigned long long s_Slev[kMaxLevels];

  const int *tok = a.tokens + static_cast<int64_t>(b) * a.N;
  const int *nxt = a.next_token + static_cast<int64_t>(b) * a.N;
  const int *sib = a.next_sibling + static_cast<int64_t>(b) * a.N;
  int rem = a.remaining ? a.remaining[b] : INT_MAX;
  if (rem < 0) rem = 0;
  int path_len = 1, n_out = 0;
  if (tid == 0) s_path[0] = 0;

  int u = 0;
  const int max_out = a.S + 1;
  while (rem > 0 && n_out < max_out) {
    const float *prow = a.target + (static_cast<int64_t>(b) * a.N + u) * V;
    if (a.mode == SDV_ACCEPT_GREEDY) {
      float bv = -INFINITY;
      int bi = INT_MAX;
      if (a.vec) {
        for (int e = lo + 4 * tid; e < hi; e += 4 * kAccThreads) {
          const float4 x = *reinterpret_cast<const float4 *>(prow + e);
          if (better(x.x, e, bv, bi)) { bv = x.x; bi = e; }
          if (better(x.y, e + 1, bv, bi)) { bv = x.y; bi = e + 1; }
          if (better(x.z, e + 2, bv, bi)) { bv = x.z; bi = e + 2; }
          if (better(x.w, e + 3, bv, bi)) { bv = x.w; bi = e + 3; }
        }
      } else {
        for (int e = lo + tid; e < hi; e += kAccThreads)
          if (better(prow[e], e, bv, bi)) { bv = prow[e]; bi = e; }
      }
      block_best(bv, bi);
      unsigned long long *slot = ring + (gen & 1) * kMaxGroup;
      if (tid == 0) store_part(slot + c, pack_best(bv, bi));
      group_barrier(ctr, gen, a.W, a.err);
      float gv = -INFINITY;
      int gi = INT_MAX;
      for (int x = 0; x < a.W; ++x) {
        const unsigned long long pk = load_part(slot + x);
        if (better(unpack_v(pk), unpack_i(pk), gv, gi)) { gv = unpack_v(pk); gi = unpack_i(pk); }
      }
      const int t = gi;
      int match = -1;
      int cc = nxt[u];
      for (int hops = 0; cc > 0 && cc < a.N && hops < a.N; ++hops) {
        if (tok[cc] == t) { match = cc; break; }
        cc = sib[cc];
      }
      if (tid == 0) s_out[n_out] = t;
      ++n_out;
      if (match >= 0) {
        if (tid == 0) s_path[path_len] = match;
        ++path_len;
      }
      if (t == a.eos || n_out == rem || match < 0) break;
      u = match;
      continue;
    }

    // ---------------- stochastic
    int qr = a.q_row[static_cast<int64_t>(b) * a.N + u];
    const bool has_kids = nxt[u] > 0 && nxt[u] < a.N && qr >= 0 && qr < a.R;
    const float *qrow = has_kids ? a.draft + (static_cast<int64_t>(b) * a.R + qr) * V : prow;
    int nlev = 0;
    int accepted = -1;
    unsigned long long last_total = 0;
    bool rejected_any = false;
    int cc = has_kids ? nxt[u] : -1;
    for (int hops = 0; cc > 0 && cc < a.N && hops < a.N && nlev < kMaxLevels; ++hops) {
      int y = tok[cc];
      y = y < 0 ? 0 : (y >= V ? V - 1 : y);
      const float qy = qrow[y];
      const float ty = t_at(prow[y], qy, s_Slev, nlev);
      const float ua = a.u_accept[static_cast<int64_t>(b) * a.N + cc];
      if (static_cast<double>(ua) * static_cast<double>(qy) < static_cast<double>(ty)) {
        accepted = cc;
        break;
      }
      // rejection: residual mass of this slice at level nlev
      unsigned long long m = 0;
      if (a.vec) {
        for (int e = lo + 4 * tid; e < hi; e += 4 * kAccThreads) {
          const float4 p4 = *reinterpret_cast<const float4 *>(prow + e);
          const float4 q4 = *reinterpret_cast<const float4 *>(qrow + e);
          m += mass_of(p4.x, q4.x, s_Slev, nlev, kResidual);
          m += mass_of(p4.y, q4.y, s_Slev, nlev, kResidual);
          m += mass_of(p4.z, q4.z, s_Slev, nlev, kResidual);
          m += mass_of(p4.w, q4.w, s_Slev, nlev, kResidual);
        }
      } else {
        for (int e = lo + tid; e < hi; e += kAccThreads) m += mass_of(prow[e], qrow[e], s_Slev, nlev, kResidual);
      }
      m = block_sum(m);
      unsigned long long *slot = ring + (gen & 1) * kMaxGroup;
      if (tid == 0) store_part(slot + c, m);
      group_barrier(ctr, gen, a.W, a.err);
      unsigned long long tot = 0;
      for (int x = 0; x < a.W; ++x) tot += load_part(slot + x);
      if (tid == 0) s_Slev[nlev] = tot;
      __syncthreads();
      ++nlev;
      last_total = tot;
      rejected_any = true;
      cc = sib[cc];
    }
    if (accepted >= 0) {
      int y = tok[accepted];
      if (tid == 0) {
        s_out[n_out] = y;
        s_path[path_len] = accepted;
      }
      ++n_out;
      ++path_len;
      if (y == a.eos || n_out == rem) break;
      u = accepted;
      continue;
    }

    // ---- draw the correction (all children rejected) or the bonus (leaf)
    int kind, lev;
    unsigned long long total;
    unsigned long long *mslot;   // slot holding the slice masses of the draw
    if (rejected_any && last_total > 0) {
      kind = kResidual;
      lev = nlev - 1;
      total = last_total;
      mslot = ring + ((gen - 1) & 1) * kMaxGroup;
    } else {
      kind = kT;
      lev = nlev;
      unsigned long long m = 0;
      for (int e = lo + tid; e < hi; e += kAccThreads) m += mass_of(prow[e], qrow[e], s_Slev, lev, kT);
      m = block_sum(m);
      mslot = ring + (gen & 1) * kMaxGroup;
      if (tid == 0) store_part(mslot + c, m);
      group_barrier(ctr, gen, a.W, a.err);
      total = 0;
      for (int x = 0; x < a.W; ++x) total += load_part(mslot + x);
    }

    int token;
    if (total == 0) {
      // degenerate: argmax of t, lowest id
      float bv = -INFINITY;
      int bi = INT_MAX;
      for (int e = lo + tid; e < hi; e += kAccThreads) {
        const float t = t_at(prow[e], qrow[e], s_Slev, lev);
        if (better(t, e, bv, bi)) { bv = t; bi = e; }
      }
      block_best(bv, bi);
      unsigned long long *slot = ring + (gen & 1) * kMaxGroup;
      if (tid == 0) store_part(slot + c, pack_best(bv, bi));
      group_barrier(ctr, gen, a.W, a.err);
      float gv = -INFINITY;
      int gi = INT_MAX;
      for (int x = 0; x < a.W; ++x) {
        const unsigned long long pk = load_part(slot + x);
        if (better(unpack_v(pk), unpack_i(pk), gv, gi)) { gv = unpack_v(pk); gi = unpack_i(pk); }
      }
      token = gi;
    } else {
      const float ud = a.u_draw[static_cast<int64_t>(b) * a.N + u];
      const unsigned long long kk = static_cast<unsigned long long>(ud * 16777216.0f);
      const unsigned long long T = kk * (total >> 24) + ((kk * (total & 0xffffffull)) >> 24);
      // the slice holding the crossing
      unsigned long long base = 0;
      int owner = a.W - 1;
      for (int x = 0; x < a.W; ++x) {
        const unsigned long long px = load_part(mslot + x);
        if (T < base + px) { owner = x; break; }
        base += px;
      }
      unsigned long long *slot = ring + (gen & 1) * kMaxGroup;
      if (c == owner) {
        // scan the slice in tiles of kE entries per thread
        constexpr int kE = 8;
        __shared__ int s_found;
        if (tid == 0) s_found = INT_MAX;
        __syncthreads();
        for (int t0 = lo; t0 < hi; t0 += kE * kAccThreads) {
          const int my0 = t0 + tid * kE;
          unsigned long long loc[kE];
          unsigned long long sum = 0;
#pragma unroll
          for (int j = 0; j < kE; ++j) {
            const int e = my0 + j;
            loc[j] = e < hi ? mass_of(prow[e], qrow[e], s_Slev, lev, kind) : 0ull;
            sum += loc[j];
          }
          unsigned long long tile_total;
          unsigned long long before = base + block_exclusive_scan(sum, tile_total);
          if (T < before + sum) {
            unsigned long long run = before;
#pragma unroll
            for (int j = 0; j < kE; ++j) {
              run += loc[j];
              if (T < run) {
                atomicMin(&s_found, my0 + j);
                break;
              }
            }
          }
          base += tile_total;
          __syncthreads();
          if (s_found != INT_MAX) break;
        }
        if (tid == 0) store_part(slot + c, static_cast<unsigned long long>(s_found == INT_MAX ? hi - 1 : s_found));
      }
      group_barrier(ctr, gen, a.W, a.err);
      token = static_cast<int>(load_part(slot + owner));
    }
    if (tid == 0) s_out[n_out] = token;
    ++n_out;
    break;
  }

  __syncthreads();
  if (c == 0) {
    for (int j = tid; j <= a.S; j += kAccThreads) {
      a.accept_path[static_cast<int64_t>(b) * (a.S + 1) + j] = j < path_len ? s_path[j] : -1;
      a.commit_tokens[static_cast<int64_t>(b) * (a.S + 1) + j] = j < n_out ? s_out[j] : -1;
    }
    if (tid == 0) {
      a.accept_len[b] = path_len - 1;
      a.commit_len[b] = n_out;
      a.next_root[b] = n_out > 0 ? s_out[n_out - 1] : -1;
    }
  }
}

__global__ void zero_u32_kernel(unsigned *p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

struct AcceptPlan {
  int W, chunk, per_launch;
};

int32_t plan_accept(const sdv_accept_shape &sh, AcceptPlan &p) {
  int per_cu = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, accept_kernel, kAccThreads, 0);
  if (e != hipSuccess || per_cu <= 0) return fail(SDV_E_HIP, "verify_accept: occupancy query failed");
  const int64_t resident = static_cast<int64_t>(per_cu) * num_cus();
  int64_t W = (2LL * num_cus()) / (sh.B > 0 ? sh.B : 1);
  const int64_t by_len = (sh.V + 1023) / 1024;
  if (W > by_len) W = by_len;
  if (W > kMaxGroup) W = kMaxGroup;
  if (W > resident) W = resident;
  if (W < 1) W = 1;
  int64_t chunk = (sh.V + W - 1) / W;
  chunk = (chunk + 3) / 4 * 4;
  p.W = static_cast<int>(W);
  p.chunk = static_cast<int>(chunk);
  int64_t per = resident / W;
  if (per < 1) per = 1;
  if (per > sh.B) per = sh.B;
  p.per_launch = static_cast<int>(per);
  return SDV_OK;
}

}  // namespace
}  // namespace sdv

using namespace sdv;

extern "C" size_t sdv_verify_accept_workspace_size(sdv_accept_shape sh) {
  if (sh.B <= 0) return 0;
  Carver c(nullptr);
  c.take<unsigned>(static_cast<size_t>(sh.B) + 1);
  c.take<unsigned long long>(static_cast<size_t>(sh.B) * 2 * kMaxGroup);
  return c.bytes();
}

extern "C" int32_t sdv_verify_accept(sdv_accept_shape sh, int32_t eos_id, const int32_t *remaining,
                                     const int32_t *tokens, const int32_t *next_token,
                                     const int32_t *next_sibling, const int32_t *q_row,
                                     const float *target, const float *draft_probs,
                                     const float *u_accept, const float *u_draw, int32_t *accept_len,
                                     int32_t *accept_path, int32_t *commit_tokens,
                                     int32_t *commit_len, int32_t *next_root, void *ws,
                                     size_t ws_bytes, void *stream) {
  clear_error();
  SDV_REQUIRE(sh.B >= 0 && sh.N >= 1 && sh.S >= 0 && sh.V >= 1, SDV_E_SHAPE,
              "verify_accept: need B >= 0, N >= 1, S >= 0, V >= 1");
  SDV_REQUIRE(sh.mode == SDV_ACCEPT_GREEDY || sh.mode == SDV_ACCEPT_STOCHASTIC, SDV_E_SHAPE,
              "verify_accept: unknown mode %d", sh.mode);
  SDV_REQUIRE(sh.N <= 256 && sh.S + 1 <= 64 && sh.V < INT_MAX - 4096, SDV_E_UNSUPPORTED,
              "verify_accept: N <= 256, S+1 <= 64 and V < 2^31-4096 required");
  SDV_REQUIRE(sh.mode == SDV_ACCEPT_GREEDY || sh.R >= 1, SDV_E_SHAPE, "verify_accept: R >= 1 needed");
  if (sh.B == 0) return SDV_OK;
  SDV_REQUIRE(tokens && next_token && next_sibling && target && accept_len && accept_path &&
                  commit_tokens && commit_len && next_root,
              SDV_E_NULL, "verify_accept: NULL pointer");
  if (sh.mode == SDV_ACCEPT_STOCHASTIC)
    SDV_REQUIRE(q_row && draft_probs && u_accept && u_draw, SDV_E_NULL,
                "verify_accept: stochastic mode needs q_row, draft_probs and uniforms");
  const size_t need = sdv_verify_accept_workspace_size(sh);
  SDV_REQUIRE(ws && ws_bytes >= need, SDV_E_WORKSPACE, "verify_accept: workspace of %zu bytes needed", need);
  AcceptPlan p;
  int32_t rc = plan_accept(sh, p);
  if (rc != SDV_OK) return rc;

  Carver cv(ws);
  unsigned *ctr = cv.take<unsigned>(static_cast<size_t>(sh.B) + 1);
  unsigned long long *part = cv.take<unsigned long long>(static_cast<size_t>(sh.B) * 2 * kMaxGroup);
  hipStream_t st = as_stream(stream);
  const int nz = sh.B + 1;
  hipLaunchKernelGGL(zero_u32_kernel, dim3((nz + 255) / 256), dim3(256), 0, st, ctr, nz);
  rc = check_launch("zero_u32_kernel");
  if (rc != SDV_OK) return rc;

  AcceptArgs a;
  a.B = sh.B; a.N = sh.N; a.S = sh.S; a.V = sh.V; a.R = sh.R; a.mode = sh.mode; a.eos = eos_id;
  a.W = p.W; a.chunk = p.chunk;
  a.vec = (sh.V % 4 == 0) && (reinterpret_cast<uintptr_t>(target) % 16 == 0) &&
          (!draft_probs || reinterpret_cast<uintptr_t>(draft_probs) % 16 == 0);
  a.remaining = remaining;
  a.tokens = tokens; a.next_token = next_token; a.next_sibling = next_sibling; a.q_row = q_row;
  a.target = target; a.draft = draft_probs; a.u_accept = u_accept; a.u_draw = u_draw;
  a.accept_len = accept_len; a.accept_path = accept_path; a.commit_tokens = commit_tokens;
  a.commit_len = commit_len; a.next_root = next_root;
  a.ctr = ctr; a.part = part; a.err = ctr + sh.B;
  for (int b0 = 0; b0 < sh.B; b0 += p.per_launch) {
    a.b0 = b0;
    const int nb = (sh.B - b0 < p.per_launch ? sh.B - b0 : p.per_launch);
    void *args[] = {&a};
    hipError_t e = hipLaunchCooperativeKernel(reinterpret_cast<const void *>(accept_kernel),
                                              dim3(static_cast<unsigned>(nb * p.W)), dim3(kAccThreads),
                                              args, 0, st);
    if (e != hipSuccess) return fail(SDV_E_HIP, "verify_accept: cooperative launch: %s", hipGetErrorString(e));
  }
  return SDV_OK;
}
