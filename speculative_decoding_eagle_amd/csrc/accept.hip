// A6-A7: target row reductions and the accept walk (zero-to-sglang ch.10
// sections 3.3, 4.1, 5.1; verify_tree_greedy and the other verification
// kernels in "EAGLE speculative decoding in four parts", "Drafting,
// verification and slots").
//
// The walk of one request is sequential in depth, but every row it reads is
// 4*V bytes, so a single wave per request cannot pull HBM bandwidth.  Each
// request is served by a group of W workgroups; workgroup c owns the
// vocabulary slice [c*T*E, (c+1)*T*E) of every row and keeps that slice of
// the current node's rows in registers (E floats per thread): the target row
// and, for rejection sampling, the draft row are read from HBM once per
// visited node, with every load of the slice in flight at once.
//
// A launch never holds more workgroups than the device keeps resident at
// once (larger batches take several launches), so every group is resident
// together.  A group exchanges a row-wide value whenever the walk needs one:
//   greedy     -- the argmax of the current node's target row;
//   stochastic -- each rejection's fixed-point residual mass (or, at a leaf,
//                 the mass of t) and, if it is zero, the argmax of t.
// Workgroup c publishes its partial as one 64-bit word that also carries the
// exchange's sequence tag, with a single agent-scope atomic store; readers
// poll the W words (lane x of each wave reads workgroup x's) until every tag
// matches.  Flag and value share one location, so no fence or counter is
// involved.  Every workgroup reduces the same W partials in the same order,
// so all of them take the same decisions.  The final inverse-CDF draw needs
// no extra exchange: the workgroup whose slice holds the crossing finds the
// token in its registers and writes the request's outputs itself.
//
// Rejection levels update t in registers as the pair (r, s): the current
// residual r = max(t - q, 0) and the scale s = S * 2^-40 of the level's mass,
// t' = fp32(double(r) / s).  These are the same operations, in the same
// order, as the single-entry recursion used for the accept test, so both
// agree bit for bit with each other and with the sampling contract.
//
// Partial words form a ring of two per request: a workgroup only publishes
// exchange n+2 after every workgroup has published exchange n+1, which each
// does only after reading exchange n.  Every poll is bounded; on timeout the
// kernel sets SDV_STATUS_ACCEPT_WAIT in the workspace header and carries on
// with fill values, so every wave always exits (the outputs of that call are
// then unspecified, and the workspace must be reset before its next use).
// The words start at zero and every call leaves them zero: when a
// workgroup has read its last word it bumps the request's counter, and the
// group's last workgroup clears the request's words and the counter, so no
// clearing launch precedes the walk.
#include <atomic>
#include <climits>
#include <cmath>
#include <mutex>

#include "common.hpp"

namespace sdv {
namespace {

constexpr int kAccThreads = 256;
constexpr int kAccWaves = kAccThreads / kWave;
constexpr int kMaxGroup = 64;          // workgroups per request
constexpr int kMaxE = 64;              // floats per thread per row slice
constexpr int kMaxLevels = 256;        // rejections at one node (children of one node)
constexpr unsigned kSpinLimit = 1u << 22;    // polls of one exchange word before giving up

struct AcceptArgs {
  int B, N, S, V, R, mode, eos;
  int W, b0;                           // group size, first request of this launch
  unsigned wait_limit;                 // polls per exchange word before giving up
  const int *remaining;
  const int *tokens, *next_token, *next_sibling, *q_row;
  const float *target, *draft, *u_accept, *u_draw;
  int *accept_len, *accept_path, *commit_tokens, *commit_len, *next_root;
  unsigned long long *part;            // [B][2][kMaxGroup] tagged partials (zero at the start, left zero)
  unsigned *done;                      // [B] workgroups of the request that have finished
  unsigned *status;                    // workspace header status word
};

// Tagged partial words.
//   argmax: value bits [63:32], tag [31:20] (12 bits), index [19:0]
//           (kNoIndex: the slice is empty);
//   mass:   tag [63:55] (9 bits), value [54:0] (a slice holds at most 2^14
//           entries of mass at most 2^40 + 2^17).
constexpr unsigned kNoIndex = 0xFFFFFu;

__device__ __forceinline__ unsigned long long pack_best(float v, int i, unsigned tag) {
  const unsigned idx = i == INT_MAX ? kNoIndex : static_cast<unsigned>(i);
  return (static_cast<unsigned long long>(__float_as_uint(v)) << 32) | ((tag & 0xFFFu) << 20) | idx;
}
__device__ __forceinline__ bool best_tag_is(unsigned long long w, unsigned tag) {
  return ((w >> 20) & 0xFFFu) == (tag & 0xFFFu);
}
__device__ __forceinline__ float unpack_v(unsigned long long w) {
  return __uint_as_float(static_cast<unsigned>(w >> 32));
}
__device__ __forceinline__ int unpack_i(unsigned long long w) {
  const unsigned idx = static_cast<unsigned>(w) & kNoIndex;
  return idx == kNoIndex ? INT_MAX : static_cast<int>(idx);
}
__device__ __forceinline__ unsigned long long pack_mass(unsigned long long m, unsigned tag) {
  return (static_cast<unsigned long long>(tag & 0x1FFu) << 55) | m;
}
__device__ __forceinline__ bool mass_tag_is(unsigned long long w, unsigned tag) {
  return (w >> 55) == (tag & 0x1FFu);
}
__device__ __forceinline__ unsigned long long unpack_mass(unsigned long long w) {
  return w & ((1ull << 55) - 1);
}

__device__ __forceinline__ void store_part(unsigned long long *p, unsigned long long v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned long long load_part(unsigned long long *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Lane x < W waits for workgroup x's word of this exchange and returns it;
// other lanes return `fill`.
template <bool MASS>
__device__ __forceinline__ unsigned long long await_part(unsigned long long *slot, int W, unsigned tag,
                                                         unsigned long long fill, unsigned limit,
                                                         unsigned *status) {
  const int x = lane_id();
  if (x >= W) return fill;
  for (unsigned spins = 0; spins < limit; ++spins) {
    const unsigned long long w = load_part(slot + x);
    if (MASS ? mass_tag_is(w, tag) : best_tag_is(w, tag)) return w;
    __builtin_amdgcn_s_sleep(1);
  }
  raise_status(status, SDV_STATUS_ACCEPT_WAIT);
  return fill;
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

// The stochastic walk holds its slices in units of 2^-40: X = x * 2^40 for
// every p, q, t and residual entry x.  The values it weighs stay in [0, 2]:
// p and q lie in [0, 1], a residual never exceeds the t it came from, and a
// rescaled residual r / S is at most 2 (S, the floored mass sum, is at least
// floor(max r * 2^40) * 2^-40 >= max r / 2).  On that range the scaling is
// exact in fp32 both ways, commutes with the rounding of t - q (a difference
// too small for a normal fp32 is exact in both units), and leaves the fp64
// quotient r / S unchanged; the mass floor(fp64(r) * 2^40) of an entry is
// floor(R), and any 64 masses (each below 2^41) sum exactly in fp64.
constexpr float kUnit = 0x1p40f;

__device__ __forceinline__ double mass_of(float X) { return floor(static_cast<double>(X)); }

// A non-negative integer below 2^53 held in a double, as a u64.
__device__ __forceinline__ unsigned long long to_u64(double m) {
  const double h = floor(m * 0x1p-32);
  return (static_cast<unsigned long long>(static_cast<unsigned>(h)) << 32) |
         static_cast<unsigned>(m - h * 0x1p32);
}

__device__ __forceinline__ unsigned long long mass(float X) { return to_u64(mass_of(X)); }

__device__ __forceinline__ float rescale(float r, double s) {
  return static_cast<float>(static_cast<double>(r) / s);
}

// T = fp32(fp64(R) / tot) * 2^40 for four entries of a slice (tot the mass
// sum as fp64, inv = fp64(2^40 / tot), both once per level).  The product
// fp64(R) * inv lies within two fp64 ulps of the quotient, hence of its
// correctly rounded value, so both round to the same fp32 unless the product
// is within a few ulps of an fp32 rounding midpoint (the 29 bits below the
// fp32 mantissa near 2^28) or t is below the fp32 normal range (the product
// below 2^-86 here); if any of the four is such a case, all four take the
// division.  R = 0 gives 0 either way.
__device__ __forceinline__ void rescale4(const float *R, float *T, double tot, double inv) {
  unsigned near = 0xFFFFFFFFu, small = 0xFFFFFFFFu;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const double qd = static_cast<double>(R[k]) * inv;
    const unsigned long long bits = __double_as_longlong(qd);
    T[k] = static_cast<float>(qd);
    near = min(near, (static_cast<unsigned>(bits) & 0x1FFFFFFFu) - (0x10000000u - 4u));
    small = min(small, static_cast<unsigned>(bits >> 32) - 1u);   // qd = 0 wraps round
  }
  // fp64 high word 0x3A900000 is 2^-86
  if (__builtin_expect(near <= 8u || small < 0x3A900000u - 1u, 0)) {
#pragma unroll
    for (int k = 0; k < 4; ++k) T[k] = rescale(R[k], tot) * kUnit;
  }
}

// t at one vocabulary entry after `lev` rejections at the current node:
// t <- fp32(double(max(t - q, 0)) / (double(S_j) * 2^-40)) for every level j
// whose residual mass S_j was non-zero.
__device__ __forceinline__ float t_at(float p, float q, const unsigned long long *Slev, int lev) {
  float t = p;
  for (int j = 0; j < lev; ++j) {
    const unsigned long long Sj = Slev[j];
    if (Sj == 0) continue;
    t = rescale(fmaxf(t - q, 0.0f), static_cast<double>(Sj) * 0x1p-40);
  }
  return t;
}

// ---------------------------------------------------------------- row slices
//
// Element x of float4 group j of thread tid is vocabulary entry
// lo + 4*(j*T + tid) + x: each load instruction of a wave covers 1 KB of
// the row, and a thread's entries ascend with (j, x).

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

template <int E, bool VEC>
__device__ __forceinline__ void load_slice(const float *__restrict__ row, int lo, int hi, float (&v)[E], float fill) {
  // recomputed at each call: kept from one call to the next, the offsets
  // and bounds would hold registers across the whole walk
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  if constexpr (VEC) {
    // A raw buffer over the slice: a load past its end returns zeros (hi - lo
    // is a multiple of 4, so a float4 lies wholly inside or outside), with
    // no address clamp and no branch, and the loads of a slice stay in
    // flight together.
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(row + lo), 0, (hi - lo) * 4, 0x00020000);
    u32x4 x[E / 4];
#pragma unroll
    for (int j = 0; j < E / 4; ++j) x[j] = __builtin_amdgcn_raw_buffer_load_b128(rs, 16 * (j * kAccThreads + tid), 0, 0);
#pragma unroll
    for (int j = 0; j < E / 4; ++j) {
      const bool ok = fill == 0.0f || lo + 4 * (j * kAccThreads + tid) < hi;
      v[4 * j + 0] = ok ? __uint_as_float(x[j].x) : fill;
      v[4 * j + 1] = ok ? __uint_as_float(x[j].y) : fill;
      v[4 * j + 2] = ok ? __uint_as_float(x[j].z) : fill;
      v[4 * j + 3] = ok ? __uint_as_float(x[j].w) : fill;
    }
  } else {
#pragma unroll
    for (int j = 0; j < E / 4; ++j)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int e = lo + 4 * (j * kAccThreads + tid) + k;
        const float y = row[e < hi ? e : lo];
        v[4 * j + k] = e < hi ? y : fill;
      }
  }
}

// Entries 4j .. 4j+3 of this thread's slice (0 past its end), as load_slice
// places them.
template <bool VEC>
__device__ __forceinline__ void load_four(const float *__restrict__ row, int lo, int hi, int j, float *v) {
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int e = lo + 4 * (j * kAccThreads + tid);
  if constexpr (VEC) {
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(row + lo), 0, (hi - lo) * 4, 0x00020000);
    const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(rs, 4 * (e - lo), 0, 0);
    v[0] = __uint_as_float(x.x);
    v[1] = __uint_as_float(x.y);
    v[2] = __uint_as_float(x.z);
    v[3] = __uint_as_float(x.w);
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = e + k < hi ? row[e + k] : 0.0f;
  }
}

// This thread's slice of `row` straight into LDS (16 bytes per lane, no
// registers): float4 j of thread t lands at q_lds[j * kAccThreads + t].  A
// lane past the slice end reads the slice's first float4 instead: the walk
// never weighs those entries (their p entry is 0, so their residual is 0
// whatever q holds there).
// The copies are issued as inline assembly (dma16), unseen by the
// compiler's wait placement, which would otherwise hold every LDS access of
// the kernel until they land; the walk waits for them itself (await_slices)
// before it first reads q_lds.
template <int E>
__device__ __forceinline__ void slice_to_lds(const float *__restrict__ row, int lo, int hi, float4 *q_lds) {
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const uint32_t wave_lds =
      lds_offset(q_lds) + static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(tid) & ~(kWave - 1)) * 16u;
#pragma unroll
  for (int j = 0; j < E / 4; ++j) {
    const int e = lo + 4 * (j * kAccThreads + tid);
    dma16(row + (e < hi ? e : lo), wave_lds + j * kAccThreads * 16u);
  }
}

// Waits for every vector-memory load this wave has in flight, the draft
// slice's LDS copy included; the memory clobber keeps LDS reads after it.
__device__ __forceinline__ void await_slices() { asm volatile("s_waitcnt vmcnt(0)" : : : "memory"); }

template <int E>
__device__ __forceinline__ int slice_index(int lo, int n) {
  return lo + 4 * ((n >> 2) * kAccThreads + static_cast<int>(threadIdx.x)) + (n & 3);
}

// Best (value, index) of the thread's entries.  Entries ascend with n and the
// out-of-slice ones come last holding -inf, so keeping the first maximum in
// n order is the (value desc, index asc) rule; a thread with no entry in the
// slice reports (-inf, INT_MAX).
template <int E>
__device__ __forceinline__ void thread_best(const float (&v)[E], int lo, int hi, float &bv, int &bi) {
  bv = v[0];
  int bn = 0;
#pragma unroll
  for (int n = 1; n < E; ++n)
    if (v[n] > bv) {
      bv = v[n];
      bn = n;
    }
  bi = slice_index<E>(lo, bn);
  if (bi >= hi) bi = INT_MAX;
}

// ------------------------------------------------------------------- kernel

__device__ void write_outputs(const AcceptArgs &a, int b, const int *s_path, const int *s_out, int path_len,
                              int n_out) {
  for (int j = threadIdx.x; j <= a.S; j += kAccThreads) {
    a.accept_path[static_cast<int64_t>(b) * (a.S + 1) + j] = j < path_len ? s_path[j] : -1;
    a.commit_tokens[static_cast<int64_t>(b) * (a.S + 1) + j] = j < n_out ? s_out[j] : -1;
  }
  if (threadIdx.x == 0) {
    a.accept_len[b] = path_len - 1;
    a.commit_len[b] = n_out;
    a.next_root[b] = n_out > 0 ? s_out[n_out - 1] : -1;
  }
}

// Keeps the compiler from interleaving the fp64 divisions of many entries
// (each holds about ten registers while in flight).
__device__ __forceinline__ void one_at_a_time() { __builtin_amdgcn_sched_barrier(0); }
// The same, except that LDS reads may move across (the next four entries'
// q is read ahead).
__device__ __forceinline__ void four_at_a_time() { __builtin_amdgcn_sched_barrier(0x0100); }

// The workgroup whose slice holds the crossing T of the running mass (lane x
// holds workgroup x's mass), and the mass of the slices before it.
__device__ __forceinline__ int group_owner(unsigned long long px, int W, unsigned long long T,
                                           unsigned long long &base) {
  unsigned long long inc = px;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const unsigned long long y = __shfl_up(inc, off, kWave);
    if (lane_id() >= off) inc += y;
  }
  const unsigned long long hit = __ballot(lane_id() < W && T < inc);
  const int owner = hit ? __ffsll(static_cast<long long>(hit)) - 1 : W - 1;
  base = __shfl(inc - px, owner, kWave);
  return owner;
}

template <int E, bool STOCH, bool VEC>
__global__ void __launch_bounds__(kAccThreads, 2) accept_kernel(AcceptArgs a) {
  const int b = a.b0 + static_cast<int>(blockIdx.x) / a.W;
  const int c = static_cast<int>(blockIdx.x) % a.W;
  if (b >= a.B) return;
  const int tid = threadIdx.x;
  const int V = a.V;
  const int N = a.N;
  constexpr int kChunk = kAccThreads * E;
  const int lo = min(V, c * kChunk);
  const int hi = min(V, lo + kChunk);
  unsigned long long *ring = a.part + static_cast<int64_t>(b) * 2 * kMaxGroup;
  unsigned gen = 0;

  __shared__ int s_path[66];
  __shared__ int s_out[66];
  __shared__ unsigned long long s_Slev[kMaxLevels];
  __shared__ int s_found;
  // the request's tree, staged once
  __shared__ int s_tok[256], s_nxt[256], s_sib[256], s_qr[256];
  __shared__ float s_ua[256];
  // children of the current node and their p[y], q[y]
  __shared__ int s_kid[256];
  __shared__ float s_py[256], s_qy[256];
  __shared__ int s_nk;

  // Slices of node u's rows, loaded where the node is chosen so that they are
  // in flight while the rest of its step is prepared: r = its target row
  // (registers); stochastic, its children's draft row goes to LDS (q_lds,
  // E KB, entry 4j+k of thread t at float4 j * kAccThreads + t): it is read
  // once per level and would otherwise hold E registers.  A node without
  // children has no levels and reads no q.
  extern __shared__ __attribute__((aligned(16))) float4 q_lds[];
  float r[E];
  auto load_q = [&](int qr, bool has_kids) {
    if constexpr (STOCH) {
      if (has_kids) {
        const float *qrow = a.draft + (static_cast<int64_t>(b) * a.R + qr) * V;
        if constexpr (VEC) {
          slice_to_lds<E>(qrow, lo, hi, q_lds);
        } else {
#pragma unroll
          for (int j = 0; j < E / 4; ++j) {
            float q4[4];
            load_four<false>(qrow, lo, hi, j, q4);
            q_lds[j * kAccThreads + tid] = make_float4(q4[0], q4[1], q4[2], q4[3]);
          }
        }
      }
    }
  };
  auto load_p = [&](int node) {
    load_slice<E, VEC>(a.target + (static_cast<int64_t>(b) * N + node) * V, lo, hi, r, STOCH ? 0.0f : -INFINITY);
  };
  // The tree (N <= kAccThreads: one node per thread) and the root's slices
  // are read together: the root's target row is known before the tree, and
  // its draft row index is read on its own.  The draft slice's copy goes
  // first, then the tree, then the target slice: the tree is then waited
  // for without waiting for the target slice.
  int rem = a.remaining ? a.remaining[b] : INT_MAX;   // (first: its wait then waits for nothing else)
  if constexpr (STOCH) {
    // a root without children has its draft row read all the same (when the
    // index is valid), and never used
    const int qr0 = a.q_row[static_cast<int64_t>(b) * N];
    load_q(qr0, qr0 >= 0 && qr0 < a.R);
  }
  int g_tok = 0, g_nxt = 0, g_sib = 0, g_qr = 0;
  float g_ua = 0.0f;
  if (tid < N) {
    const int64_t g = static_cast<int64_t>(b) * N + tid;
    g_tok = a.tokens[g];
    g_nxt = a.next_token[g];
    g_sib = a.next_sibling[g];
    if constexpr (STOCH) {
      g_qr = a.q_row[g];
      g_ua = a.u_accept[g];
    }
  }
  load_p(0);
  if (tid < N) {
    s_tok[tid] = g_tok;
    s_nxt[tid] = g_nxt;
    s_sib[tid] = g_sib;
    if constexpr (STOCH) {
      s_qr[tid] = g_qr;
      s_ua[tid] = g_ua;
    }
  }
  if (tid == 0) s_path[0] = 0;
  if (rem < 0) rem = 0;
  __syncthreads();

  // Exchanges: publish this workgroup's partial, then every wave gathers the
  // group's partials (lane x: workgroup x).
  auto group_best = [&](float v, int i) -> int {
    block_best(v, i);
    unsigned long long *slot = ring + (gen & 1) * kMaxGroup;
    ++gen;
    if (tid == 0) store_part(slot + c, pack_best(v, i, gen));
    const unsigned long long w =
        await_part<false>(slot, a.W, gen, pack_best(-INFINITY, INT_MAX, gen), a.wait_limit, a.status);
    float gv = unpack_v(w);
    int gi = unpack_i(w);
    wave_best(gv, gi);
    return gi;
  };
  // returns the group total; `lane_mass` receives workgroup lane_id()'s part
  auto group_mass = [&](unsigned long long m, unsigned long long &lane_mass) -> unsigned long long {
    m = block_sum(m);
    unsigned long long *slot = ring + (gen & 1) * kMaxGroup;
    ++gen;
    if (tid == 0) store_part(slot + c, pack_mass(m, gen));
    lane_mass = unpack_mass(await_part<true>(slot, a.W, gen, pack_mass(0, gen), a.wait_limit, a.status));
    return wave_sum_u64(lane_mass);
  };

  int path_len = 1, n_out = 0;
  bool writer = c == 0;
  int u = 0;
  const int max_out = a.S + 1;
  while (rem > 0 && n_out < max_out) {
    const float *prow = a.target + (static_cast<int64_t>(b) * N + u) * V;
    if constexpr (!STOCH) {
      float bv;
      int bi;
      thread_best<E>(r, lo, hi, bv, bi);
      const int t = group_best(bv, bi);
      int match = -1;
      int cc = s_nxt[u];
      for (int hops = 0; cc > 0 && cc < N && hops < N; ++hops) {
        if (s_tok[cc] == t) {
          match = cc;
          break;
        }
        cc = s_sib[cc];
      }
      if (tid == 0) s_out[n_out] = t;
      ++n_out;
      if (match >= 0) {
        if (tid == 0) s_path[path_len] = match;
        ++path_len;
      }
      if (t == a.eos || n_out == rem || match < 0) break;
      u = match;
      load_p(u);
      continue;
    } else {
      // ---------------- stochastic: t is held as (r, s); level 0 is t = p
      const int qr = s_qr[u];
      const bool has_kids = s_nxt[u] > 0 && s_nxt[u] < N && qr >= 0 && qr < a.R;
      const float *qrow = has_kids ? a.draft + (static_cast<int64_t>(b) * a.R + qr) * V : prow;
      if (tid == 0) {
        int nk = 0;
        int cc = has_kids ? s_nxt[u] : -1;
        for (int hops = 0; cc > 0 && cc < N && hops < N && nk < kMaxLevels; ++hops) {
          s_kid[nk++] = cc;
          cc = s_sib[cc];
        }
        s_nk = nk;
      }
      __syncthreads();
      const int nk = s_nk;
      for (int i = tid; i < nk; i += kAccThreads) {
        int y = s_tok[s_kid[i]];
        y = y < 0 ? 0 : (y >= V ? V - 1 : y);
        s_py[i] = prow[y];
        s_qy[i] = qrow[y];
      }
      __syncthreads();
      // r holds t itself (scaled false: the row p, or t rebuilt after a level
      // of zero mass), or the last residual R in units of 2^-40, with
      // T = R / tot (scaled true)
      bool scaled = false;
      double tot_d = 1.0, inv = 1.0;
      int nlev = 0;
      int accepted = -1;
      unsigned long long last_total = 0;
      unsigned long long last_lane = 0;
      for (int i = 0; i < nk; ++i) {
        const int cc = s_kid[i];
        const float qy = s_qy[i];
        const float ty = t_at(s_py[i], qy, s_Slev, nlev);
        if (static_cast<double>(s_ua[cc]) * static_cast<double>(qy) < static_cast<double>(ty)) {
          accepted = cc;
          break;
        }
        // rejection: r <- max(t - q, 0) and its mass
        if (nlev == 0) await_slices();
        // (T - q * 2^40 as one fma: the product is exact, so this is the
        // rounded difference in units of 2^-40)
        double m = 0.0;
        if (scaled) {
#pragma unroll
          for (int g = 0; g < E / 4; ++g) {
            const float4 q4 = q_lds[g * kAccThreads + tid];
            const float qg[4] = {q4.x, q4.y, q4.z, q4.w};
            float T[4];
            rescale4(&r[4 * g], T, tot_d, inv);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              r[4 * g + k] = fmaxf(fmaf(qg[k], -kUnit, T[k]), 0.0f);
              m += mass_of(r[4 * g + k]);
            }
            four_at_a_time();
          }
        } else {
          // t * 2^40 - q * 2^40, both products exact
#pragma unroll
          for (int g = 0; g < E / 4; ++g) {
            const float4 q4 = q_lds[g * kAccThreads + tid];
            const float qg[4] = {q4.x, q4.y, q4.z, q4.w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              r[4 * g + k] = fmaxf(fmaf(r[4 * g + k], kUnit, qg[k] * -kUnit), 0.0f);
              m += mass_of(r[4 * g + k]);
            }
            four_at_a_time();
          }
        }
        unsigned long long lane_mass;
        const unsigned long long tot = group_mass(to_u64(m), lane_mass);
        if (tid == 0) s_Slev[nlev] = tot;
        __syncthreads();
        ++nlev;
        last_total = tot;
        last_lane = lane_mass;
        if (tot > 0) {
          scaled = true;
          tot_d = static_cast<double>(tot);
          inv = 0x1p40 / tot_d;
        } else {
          // A level of zero mass leaves t as it was, but r already holds its
          // residual: rebuild t from the row through the levels so far (rare).
          // (four entries at a time, to hold few registers on this path)
#pragma unroll
          for (int j = 0; j < E / 4; ++j) {
            float p4[4];
            load_four<VEC>(prow, lo, hi, j, p4);
            const float4 q4 = q_lds[j * kAccThreads + tid];
            const float qg[4] = {q4.x, q4.y, q4.z, q4.w};
#pragma unroll
            for (int k = 0; k < 4; ++k) r[4 * j + k] = t_at(p4[k], qg[k], s_Slev, nlev);
            one_at_a_time();
          }
          scaled = false;
        }
      }
      if (accepted >= 0) {
        const int y = s_tok[accepted];
        if (tid == 0) {
          s_out[n_out] = y;
          s_path[path_len] = accepted;
        }
        ++n_out;
        ++path_len;
        if (y == a.eos || n_out == rem) break;
        u = accepted;
        {
          const int nqr = s_qr[u];
          load_q(nqr, s_nxt[u] > 0 && s_nxt[u] < N && nqr >= 0 && nqr < a.R);
          load_p(u);
        }
        __syncthreads();             // s_kid / s_py / s_qy are rewritten for the next node
        continue;
      }

      // ---- draw the correction (all children rejected) or the bonus (leaf):
      // from the last residual if its mass is non-zero, else from t
      const bool from_residual = nlev > 0 && last_total > 0;
      unsigned long long lane_mass;
      unsigned long long total;
      if (from_residual) {
        lane_mass = last_lane;
        total = last_total;
      } else {
        // t itself (a leaf's bonus, or every residual of zero mass), to
        // units of 2^-40
        if (scaled) {
#pragma unroll
          for (int g = 0; g < E / 4; ++g) {
            float T[4];
            rescale4(&r[4 * g], T, tot_d, inv);
#pragma unroll
            for (int k = 0; k < 4; ++k) r[4 * g + k] = T[k];
            one_at_a_time();
          }
          scaled = false;
        } else {
#pragma unroll
          for (int n = 0; n < E; ++n) r[n] *= kUnit;
        }
        double m = 0.0;
#pragma unroll
        for (int n = 0; n < E; ++n) {
          m += mass_of(r[n]);
          if ((n & 3) == 3) one_at_a_time();
        }
        total = group_mass(to_u64(m), lane_mass);
      }

      if (total == 0) {
        // degenerate: argmax of t, lowest id (r holds t, in units of 2^-40)
        float bv;
        int bi;
        thread_best<E>(r, lo, hi, bv, bi);
        const int token = group_best(bv, bi);
        if (tid == 0) s_out[n_out] = token;
        ++n_out;
        break;
      }

      const float ud = a.u_draw[static_cast<int64_t>(b) * N + u];
      const unsigned long long kk = static_cast<unsigned long long>(ud * 16777216.0f);
      const unsigned long long T = kk * (total >> 24) + ((kk * (total & 0xffffffull)) >> 24);
      unsigned long long base;
      const int owner = group_owner(lane_mass, a.W, T, base);
      if (c != owner) {
        writer = false;
        break;
      }
      writer = true;
      // masses of the drawn distribution, scanned in vocabulary order: group j
      // of every thread, then the next group
      if (tid == 0) s_found = INT_MAX;
      __syncthreads();
#pragma unroll
      for (int j = 0; j < E / 4; ++j) {
        unsigned long long w4[4];
        unsigned long long sum = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int n = 4 * j + k;
          w4[k] = mass(r[n]);
          sum += w4[k];
          if (k == 3) one_at_a_time();
        }
        unsigned long long grp_total;
        const unsigned long long before = base + block_exclusive_scan(sum, grp_total);
        if (T >= before && T < before + sum) {
          unsigned long long run = before;
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            run += w4[k];
            if (T < run) {
              s_found = slice_index<E>(lo, 4 * j + k);
              break;
            }
          }
        }
        base += grp_total;
        __syncthreads();
        if (s_found != INT_MAX) break;
      }
      const int token = s_found == INT_MAX ? hi - 1 : s_found;
      if (tid == 0) s_out[n_out] = token;
      ++n_out;
      break;
    }
  }

  __syncthreads();
  if (writer) write_outputs(a, b, s_path, s_out, path_len, n_out);
  // Every wave of this workgroup is past its last read of the ring (the
  // barrier above: the values read have been used); the group's last
  // workgroup to get here clears it, one word per thread.  No fence is
  // needed: no read of the ring is outstanding in any workgroup that has
  // counted itself, and the clearing stores need only land before the next
  // call's launch.
  __shared__ int s_last;
  if (tid == 0) {
    const unsigned prev = __hip_atomic_fetch_add(a.done + b, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = prev == static_cast<unsigned>(a.W - 1);
  }
  __syncthreads();
  if (s_last) {
    if (tid < 2 * kMaxGroup) store_part(ring + tid, 0ull);
    if (tid == 0) __hip_atomic_store(a.done + b, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

struct AcceptPlan {
  int W, E, per_launch;
};

template <int E>
const void *kernel_of(bool stoch, bool vec) {
  if (stoch)
    return vec ? reinterpret_cast<const void *>(accept_kernel<E, true, true>)
               : reinterpret_cast<const void *>(accept_kernel<E, true, false>);
  return vec ? reinterpret_cast<const void *>(accept_kernel<E, false, true>)
             : reinterpret_cast<const void *>(accept_kernel<E, false, false>);
}

const void *accept_kernel_for(int E, bool stoch, bool vec) {
  switch (E) {
    case 4: return kernel_of<4>(stoch, vec);
    case 8: return kernel_of<8>(stoch, vec);
    case 16: return kernel_of<16>(stoch, vec);
    case 32: return kernel_of<32>(stoch, vec);
    default: return kernel_of<64>(stoch, vec);
  }
}

// Dynamic LDS of a variant: the stochastic walk keeps the draft slice there.
size_t accept_lds(int E, bool stoch) { return stoch ? static_cast<size_t>(E) * kAccThreads * sizeof(float) : 0; }

// Resident workgroups per CU of one kernel variant, queried once per device
// (which also raises the variant's dynamic LDS limit on that device).
int32_t blocks_per_cu(int E, bool stoch, bool vec, int &per_cu) {
  constexpr int kDevices = 64;
  static std::atomic<int> cache[kDevices][5][2][2];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(SDV_E_HIP, "verify_accept: no device");
  if (dev < 0 || dev >= kDevices) return fail(SDV_E_UNSUPPORTED, "verify_accept: device %d", dev);
  int ei = 0;
  while ((4 << ei) < E) ++ei;
  std::atomic<int> *slot = &cache[dev][ei][stoch][vec];
  per_cu = slot->load(std::memory_order_relaxed);
  if (per_cu > 0) return SDV_OK;
  const void *fn = accept_kernel_for(E, stoch, vec);
  const size_t lds = accept_lds(E, stoch);
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
  if (e != hipSuccess) return fail(SDV_E_HIP, "verify_accept: LDS attribute: %s", hipGetErrorString(e));
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kAccThreads, lds);
  if (e != hipSuccess || per_cu <= 0) return fail(SDV_E_HIP, "verify_accept: occupancy query failed");
  slot->store(per_cu, std::memory_order_relaxed);
  return SDV_OK;
}

// Group size: enough workgroups to cover one per CU over the batch (two per
// CU measured 1.2 us slower at 32 requests: more words per exchange, slices
// no faster to read), no more than the vocabulary needs at 4 floats per
// thread, and at least what it needs at kMaxE floats per thread; the slice
// width E then follows.
int32_t plan_accept(const sdv_accept_shape &sh, bool vec, AcceptPlan &p) {
  const int64_t T = kAccThreads;
  int64_t W = (static_cast<int64_t>(num_cus()) + sh.B - 1) / (sh.B > 0 ? sh.B : 1);
  const int64_t w_small = (sh.V + T * 4 - 1) / (T * 4);
  const int64_t w_big = (sh.V + T * kMaxE - 1) / (T * kMaxE);
  if (W > w_small) W = w_small;
  if (W > kMaxGroup) W = kMaxGroup;
  if (W < w_big) W = w_big;
  if (W < 1) W = 1;
  int E = 4;
  while (E < kMaxE && T * E * W < sh.V) E <<= 1;
  W = (sh.V + T * E - 1) / (T * E);       // no empty slices
  int per_cu = 0;
  const int32_t rc = blocks_per_cu(E, sh.mode == SDV_ACCEPT_STOCHASTIC, vec, per_cu);
  if (rc != SDV_OK) return rc;
  const int64_t resident = static_cast<int64_t>(per_cu) * num_cus();
  if (W > resident) return fail(SDV_E_UNSUPPORTED, "verify_accept: group of %lld workgroups cannot be resident",
                                static_cast<long long>(W));
  int64_t per = resident / W;
  if (per > sh.B) per = sh.B;
  p.W = static_cast<int>(W);
  p.E = E;
  p.per_launch = static_cast<int>(per);
  return SDV_OK;
}

}  // namespace
}  // namespace sdv

using namespace sdv;

extern "C" size_t sdv_verify_accept_workspace_size(sdv_accept_shape sh) {
  if (sh.B <= 0) return 0;
  Carver c(nullptr);
  c.take<char>(kWsHeaderBytes);
  c.take<unsigned long long>(static_cast<size_t>(sh.B) * 2 * kMaxGroup);
  c.take<unsigned>(static_cast<size_t>(sh.B));
  return c.bytes();
}

namespace sdv {
namespace {

int32_t run_accept(sdv_accept_shape sh, int32_t eos_id, const int32_t *remaining, const int32_t *tokens,
                   const int32_t *next_token, const int32_t *next_sibling, const int32_t *q_row,
                   const float *target, const float *draft_probs, const float *u_accept, const float *u_draw,
                   int32_t *accept_len, int32_t *accept_path, int32_t *commit_tokens, int32_t *commit_len,
                   int32_t *next_root, void *ws, size_t ws_bytes, void *stream) {
  SDV_REQUIRE(sh.B >= 0 && sh.N >= 1 && sh.S >= 0 && sh.V >= 1, SDV_E_SHAPE,
              "verify_accept: need B >= 0, N >= 1, S >= 0, V >= 1");
  SDV_REQUIRE(sh.mode == SDV_ACCEPT_GREEDY || sh.mode == SDV_ACCEPT_STOCHASTIC, SDV_E_SHAPE,
              "verify_accept: unknown mode %d", sh.mode);
  SDV_REQUIRE(sh.N <= 256 && sh.S + 1 <= 64 && sh.V < static_cast<int>(kNoIndex), SDV_E_UNSUPPORTED,
              "verify_accept: N <= 256, S+1 <= 64 and V < %d required", static_cast<int>(kNoIndex));
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
  const bool vec = (sh.V % 4 == 0) && (reinterpret_cast<uintptr_t>(target) % 16 == 0) &&
                   (!draft_probs || reinterpret_cast<uintptr_t>(draft_probs) % 16 == 0);
  AcceptPlan p;
  int32_t rc = plan_accept(sh, vec, p);
  if (rc != SDV_OK) return rc;

  Carver cv(ws);
  unsigned *header = reinterpret_cast<unsigned *>(cv.take<char>(kWsHeaderBytes));
  unsigned long long *part = cv.take<unsigned long long>(static_cast<size_t>(sh.B) * 2 * kMaxGroup);
  unsigned *done = cv.take<unsigned>(static_cast<size_t>(sh.B));
  hipStream_t st = as_stream(stream);

  AcceptArgs a;
  a.B = sh.B; a.N = sh.N; a.S = sh.S; a.V = sh.V; a.R = sh.R; a.mode = sh.mode; a.eos = eos_id;
  a.W = p.W;
  a.remaining = remaining;
  a.tokens = tokens; a.next_token = next_token; a.next_sibling = next_sibling; a.q_row = q_row;
  a.target = target; a.draft = draft_probs; a.u_accept = u_accept; a.u_draw = u_draw;
  a.accept_len = accept_len; a.accept_path = accept_path; a.commit_tokens = commit_tokens;
  a.commit_len = commit_len; a.next_root = next_root;
  a.part = part;
  a.done = done;
  a.status = header + kWsStatus;
  a.wait_limit = wait_limit(kSpinLimit);
  const void *fn = accept_kernel_for(p.E, sh.mode == SDV_ACCEPT_STOCHASTIC, vec);
  for (int b0 = 0; b0 < sh.B; b0 += p.per_launch) {
    a.b0 = b0;
    const int nb = (sh.B - b0 < p.per_launch ? sh.B - b0 : p.per_launch);
    void *args[] = {&a};
    hipError_t e = hipLaunchKernel(fn, dim3(static_cast<unsigned>(nb * p.W)), dim3(kAccThreads), args,
                                   accept_lds(p.E, sh.mode == SDV_ACCEPT_STOCHASTIC), st);
    if (e != hipSuccess) return fail(SDV_E_HIP, "verify_accept: launch: %s", hipGetErrorString(e));
  }
  return SDV_OK;
}

// ------------------------------------------------ the no-allocation variant
//
// The exchange words, counters and header of up to kNoAllocMaxB requests
// live in a file-scope device array, one copy per device that runs the
// library, held until the process ends.  In host code `scratch` only names
// the symbol: its device address is looked up once per device with
// hipGetSymbolAddress and kept in g_scratch_addr.
constexpr int kNoAllocMaxB = 1024;
constexpr size_t kNoAllocBytes = kWsHeaderBytes + static_cast<size_t>(kNoAllocMaxB) * 2 * kMaxGroup * 8 +
                                 static_cast<size_t>(kNoAllocMaxB) * 4;
static_assert(kNoAllocBytes % 256 == 0, "scratch regions are 256-byte aligned");

__device__ __align__(256) unsigned char scratch[kNoAllocBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_addr[kMaxDevices] = {};

__global__ void zero_scratch_kernel(unsigned *p, size_t n) {
  const size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// Device address of this device's copy of `scratch` (looked up on the
// first call on the device, with that device current).
int32_t scratch_address(void **out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(SDV_E_HIP, "verify_accept_noalloc: no device");
  if (dev < 0 || dev >= kMaxDevices) return fail(SDV_E_UNSUPPORTED, "verify_accept_noalloc: device %d", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void *ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(SDV_E_HIP, "verify_accept_noalloc: hipGetSymbolAddress: %s", hipGetErrorString(e));
    g_scratch_addr[dev] = ptr;
  }
  *out = g_scratch_addr[dev];
  return SDV_OK;
}

}  // namespace
}  // namespace sdv

extern "C" int32_t sdv_verify_accept(sdv_accept_shape sh, int32_t eos_id, const int32_t *remaining,
                                     const int32_t *tokens, const int32_t *next_token,
                                     const int32_t *next_sibling, const int32_t *q_row,
                                     const float *target, const float *draft_probs,
                                     const float *u_accept, const float *u_draw, int32_t *accept_len,
                                     int32_t *accept_path, int32_t *commit_tokens,
                                     int32_t *commit_len, int32_t *next_root, void *ws,
                                     size_t ws_bytes, void *stream) {
  clear_error();
  return run_accept(sh, eos_id, remaining, tokens, next_token, next_sibling, q_row, target, draft_probs, u_accept,
                    u_draw, accept_len, accept_path, commit_tokens, commit_len, next_root, ws, ws_bytes, stream);
}

extern "C" int32_t sdv_verify_accept_noalloc(sdv_accept_shape sh, int32_t eos_id, const int32_t *remaining,
                                             const int32_t *tokens, const int32_t *next_token,
                                             const int32_t *next_sibling, const int32_t *q_row,
                                             const float *target, const float *draft_probs,
                                             const float *u_accept, const float *u_draw, int32_t *accept_len,
                                             int32_t *accept_path, int32_t *commit_tokens, int32_t *commit_len,
                                             int32_t *next_root, void *stream) {
  clear_error();
  SDV_REQUIRE(sh.B <= kNoAllocMaxB, SDV_E_UNSUPPORTED,
              "verify_accept_noalloc: B=%d above the %d requests its static scratch holds", sh.B, kNoAllocMaxB);
  if (sh.B <= 0) return run_accept(sh, eos_id, remaining, tokens, next_token, next_sibling, q_row, target,
                                   draft_probs, u_accept, u_draw, accept_len, accept_path, commit_tokens,
                                   commit_len, next_root, nullptr, 0, stream);
  void *ptr = nullptr;
  int32_t rc = scratch_address(&ptr);
  if (rc != SDV_OK) return rc;
  const size_t need = sdv_verify_accept_workspace_size(sh);
  SDV_REQUIRE(need <= kNoAllocBytes, SDV_E_UNSUPPORTED, "verify_accept_noalloc: %zu scratch bytes needed", need);
  // the part of the scratch this call uses starts at zero (a wait that gave
  // up in an earlier call may have left words behind); a fill kernel, no
  // memset node, so that the call can be captured
  const size_t words = need / sizeof(unsigned);
  hipLaunchKernelGGL(zero_scratch_kernel, dim3(static_cast<unsigned>((words + 255) / 256)), dim3(256), 0,
                     as_stream(stream), static_cast<unsigned *>(ptr), words);
  rc = check_launch("verify_accept_noalloc: clear");
  if (rc != SDV_OK) return rc;
  return run_accept(sh, eos_id, remaining, tokens, next_token, next_sibling, q_row, target, draft_probs, u_accept,
                    u_draw, accept_len, accept_path, commit_tokens, commit_len, next_root, ptr, need, stream);
}
