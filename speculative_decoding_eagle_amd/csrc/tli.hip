// A9-A10: Token-Level Intersection for heterogeneous vocabularies (sglang PR
// #22883 "TLI (Token-Level Intersection)", "Modifications"): the pruned
// draft LM head, the vocabulary maps, the logit constraint and the scatter
// of the draft distribution into the target vocabulary.
//
// The pruned LM head is a skinny GEMM (B ~ 64 rows) that streams the
// [K, H] bf16 weight once from HBM with bf16 MFMA 16x16x32 and fp32
// accumulators over all B rows.  Where the hidden rows of a pass fit in LDS
// (B <= 64 and up to about 160 KB), a block of 15 waves stages them there
// once and each wave streams 16 weight rows, reading its hidden fragments
// from LDS: 240 weight rows per block, 250 blocks at K = 60000 (a CU each).
// Otherwise each 4-wave block owns 256 weight rows, each wave 64 of them,
// and the hidden fragments come from L1/L2, each serving four weight
// fragments.  (Measured at B=64, H=896, K=60000 on MI355X: 25.5 us staged
// against 35 us; without the LDS, more waves per CU ran slower -- 44 us with
// 32 weight rows per wave, 67 with 16 -- since every wave re-reads the
// hidden matrix per weight fragment.)  The constraint writes 16 bytes
// per thread and row over eight rows per block, its gathers all in flight;
// the scatter passes each q row through LDS so that its random gathers
// read LDS; the id maps are coalesced gathers/scatters.
#include <algorithm>
#include <cmath>

#include "common.hpp"

namespace sdv {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef float f32x4v __attribute__((ext_vector_type(4)));
constexpr int kRowsPerScatter = 8;   // rows per block of the 4-wide scatter and constraint kernels
constexpr int kXcdCount = 8;

constexpr int kGemmThreads = 256;
constexpr int kNBlocks = 4;         // 16-row weight blocks per wave
constexpr int kRowsPerBlock = kGemmThreads / 64 * 16 * kNBlocks;   // weight rows (output columns) per block
constexpr int kMaxMBlocks = 8;      // hidden rows handled per pass: 8 x 16 = 128

__device__ __forceinline__ bf16x8 load_bf16x8(const uint16_t *p) {
  const uint4 u = *reinterpret_cast<const uint4 *>(p);
  bf16x8 r;
  __builtin_memcpy(&r, &u, sizeof(r));
  return r;
}

// logits[b, j] = sum_h hidden[b, h] * weight[j, h].  Wave w of a block owns
// NB blocks of 16 weight rows; per 32-column step it loads NB weight and MB
// hidden fragments (16 bytes per lane each) and runs NB * MB MFMAs, so each
// hidden fragment read from L1/L2 serves NB weight fragments.
template <int MB, int NB>
__global__ void __launch_bounds__(kGemmThreads)
lm_head_kernel(int B, int H, int K, const uint16_t *__restrict__ hidden,
               const uint16_t *__restrict__ weight, float *__restrict__ logits) {
  const int wave = threadIdx.x / kWave;
  const int l = lane_id();
  const int n0 = (blockIdx.x * (kGemmThreads / kWave) + wave) * (16 * NB);   // first weight row of this wave
  const int m0 = blockIdx.y * (MB * 16);                                     // first hidden row of this pass
  const int kofs = 8 * (l >> 4);
  const uint16_t *wp[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int nrow = min(n0 + nb * 16 + (l & 15), K - 1);                   // clamp the tail (never stored)
    wp[nb] = weight + static_cast<int64_t>(nrow) * H + kofs;
  }
  const uint16_t *hp[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int mrow = min(m0 + mb * 16 + (l & 15), B - 1);
    hp[mb] = hidden + static_cast<int64_t>(mrow) * H + kofs;
  }
  f32x4 acc[MB][NB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int k0 = 0; k0 < H; k0 += 32) {
    bf16x8 bw[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) bw[nb] = load_bf16x8(wp[nb] + k0);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const bf16x8 ah = load_bf16x8(hp[mb] + k0);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bw[nb], acc[mb][nb], 0, 0, 0);
    }
  }
  // D[m][n]: lane l holds rows 4*(l/16)+i of the 16x16 block, column l%16
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int ncol = n0 + nb * 16 + (l & 15);
    if (ncol >= K) continue;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = m0 + mb * 16 + 4 * (l >> 4) + i;
        if (m < B) logits[static_cast<int64_t>(m) * K + ncol] = acc[mb][nb][i];
      }
  }
}

// The same product with the pass's hidden rows staged in LDS: NW waves of 16
// weight rows each; the rows of the stage are padded by kHPad bf16 so that
// the 16 rows of one fragment read fall in distinct banks.  The first kPre
// k-steps of weight fragments are issued before the staging so that the
// weight stream starts at once.  Dynamic LDS: MB * 16 * (H + kHPad) * 2
// bytes.
constexpr int kHPad = 8;
constexpr int kLdsWaves = 15;                  // 240 weight rows per block
constexpr int kLdsMax = 160 * 1024;            // staged hidden rows at most (bytes)
template <int MB, int NW>
__global__ void __launch_bounds__(NW * 64)
lm_head_lds_kernel(int B, int H, int K, const uint16_t *__restrict__ hidden,
                   const uint16_t *__restrict__ weight, float *__restrict__ logits) {
  extern __shared__ __attribute__((aligned(16))) uint16_t s_h[];
  const int wave = threadIdx.x / kWave;
  const int l = lane_id();
  const int tid = threadIdx.x;
  const int HP = H + kHPad;
  const int n0 = (blockIdx.x * NW + wave) * 16;            // first weight row of this wave
  const int m0 = blockIdx.y * (MB * 16);                   // first hidden row of this pass
  const int kofs = 8 * (l >> 4);
  const uint16_t *wp = weight + static_cast<int64_t>(min(n0 + (l & 15), K - 1)) * H + kofs;   // tail rows clamped, never stored
  constexpr int kPre = 8;
  bf16x8 pre[kPre];
#pragma unroll
  for (int p = 0; p < kPre; ++p) pre[p] = load_bf16x8(wp + min(32 * p, H - 32));
  for (int i = 8 * tid; i < MB * 16 * H; i += NW * 64 * 8) {
    const int r = i / H, col = i - r * H;                  // H % 32 == 0: a chunk stays in its row
    uint4 u = make_uint4(0, 0, 0, 0);
    if (m0 + r < B) u = *reinterpret_cast<const uint4 *>(hidden + static_cast<int64_t>(m0 + r) * H + col);
    *reinterpret_cast<uint4 *>(s_h + r * HP + col) = u;
  }
  __syncthreads();
  f32x4 acc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
  const uint16_t *hl = s_h + (l & 15) * HP + kofs;
  auto kstep = [&](int k0, const bf16x8 &bw) __attribute__((always_inline)) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      bf16x8 ah;
      const uint4 u = *reinterpret_cast<const uint4 *>(hl + mb * 16 * HP + k0);
      __builtin_memcpy(&ah, &u, 16);
      acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bw, acc[mb], 0, 0, 0);
    }
  };
#pragma unroll
  for (int p = 0; p < kPre; ++p)
    if (32 * p < H) kstep(32 * p, pre[p]);
#pragma unroll 4
  for (int k0 = 32 * kPre; k0 < H; k0 += 32) kstep(k0, load_bf16x8(wp + k0));
  // D[m][n]: lane l holds rows 4*(l/16)+i of the 16x16 block, column l%16
  const int ncol = n0 + (l & 15);
  if (ncol >= K) return;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = m0 + mb * 16 + 4 * (l >> 4) + i;
      if (m < B) logits[static_cast<int64_t>(m) * K + ncol] = acc[mb][i];
    }
}

__global__ void fill_i32_kernel(int *p, int64_t n, int v) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

__global__ void scatter_maps_kernel(int K, const int *__restrict__ inter, const int *__restrict__ tgt,
                                    int Vd, int Vt, int *__restrict__ d2t, int *__restrict__ t2d) {
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= K) return;
  const int d = inter[j], t = tgt[j];
  if (d >= 0 && d < Vd) d2t[d] = (t >= 0 && t < Vt) ? t : -1;
  if (t >= 0 && t < Vt && d >= 0 && d < Vd) t2d[t] = d;
}

__global__ void map_ids_kernel(const int *__restrict__ table, int len, const int *__restrict__ ids, int64_t n,
                               int *__restrict__ out) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int x = ids[i];
  out[i] = (x >= 0 && x < len) ? table[x] : -1;
}

// Position of v in the sorted list, or -1.
__device__ __forceinline__ int find_sorted(const int *__restrict__ a, int n, int v) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (a[mid] < v) lo = mid + 1; else hi = mid;
  }
  return (lo < n && a[lo] == v) ? lo : -1;
}

// Four consecutive draft ids per thread: one search finds the first, the
// sorted list gives the other three by stepping; kRowsPerScatter rows per
// block, 16-byte non-temporal stores.  Needs Vd % 4 == 0 and a 16-byte
// aligned output.
__global__ void __launch_bounds__(256)
constrain4_kernel(int B, int K, int Vd, const float *__restrict__ pruned, const int *__restrict__ inter,
                  float *__restrict__ full) {
  const int v = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (v >= Vd) return;
  int lo = 0, hi = K;                    // first position with inter[pos] >= v
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (inter[mid] < v) lo = mid + 1; else hi = mid;
  }
  int j[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const bool hit = lo < K && inter[lo] == v + q;
    j[q] = hit ? lo : -1;
    lo += hit ? 1 : 0;
  }
  const int b0 = blockIdx.y * kRowsPerScatter;
#pragma unroll
  for (int bb = 0; bb < kRowsPerScatter; ++bb) {
    const int b = b0 + bb;
    if (b >= B) break;
    const float *pr = pruned + static_cast<int64_t>(b) * K;
    f32x4v o;
    o.x = j[0] >= 0 ? pr[j[0]] : -INFINITY;
    o.y = j[1] >= 0 ? pr[j[1]] : -INFINITY;
    o.z = j[2] >= 0 ? pr[j[2]] : -INFINITY;
    o.w = j[3] >= 0 ? pr[j[3]] : -INFINITY;
    __builtin_nontemporal_store(o, reinterpret_cast<f32x4v *>(full + static_cast<int64_t>(b) * Vd + v));
  }
}

__global__ void constrain_kernel(int B, int K, int Vd, const float *__restrict__ pruned,
                                 const int *__restrict__ inter, float *__restrict__ full) {
  const int v = blockIdx.x * blockDim.x + threadIdx.x;
  if (v >= Vd) return;
  const int j = find_sorted(inter, K, v);
  for (int b = 0; b < B; ++b)
    full[static_cast<int64_t>(b) * Vd + v] = j >= 0 ? pruned[static_cast<int64_t>(b) * K + j] : -INFINITY;
}

// inv[tgt[j]] = j (target ids outside [0, Vt) are skipped); the header
// records K and Vt so that a later call without ids can check it is reusing
// the same map.
__global__ void inverse_kernel(int K, const int *__restrict__ tgt, int Vt, int *__restrict__ inv,
                               unsigned *__restrict__ hdr) {
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j == 0) {
    hdr[kWsStatus] = 0u;                 // a fresh map: no earlier status applies
    hdr[kWsTliK] = static_cast<unsigned>(K);
    hdr[kWsTliV] = static_cast<unsigned>(Vt);
    hdr[kWsTliMagic] = kTliMagic;
  }
  if (j >= K) return;
  const int t = tgt[j];
  if (t >= 0 && t < Vt) inv[t] = j;
}

// True when the workspace's inverse was built for this K and Vt; otherwise
// the call reports SDV_STATUS_TLI_REUSE (once per workgroup) and the caller
// gets zeros instead of a gather through a foreign map.
__device__ __forceinline__ bool map_matches(unsigned *hdr, int K, int Vt) {
  const bool ok = hdr[kWsTliK] == static_cast<unsigned>(K) && hdr[kWsTliV] == static_cast<unsigned>(Vt) &&
                  hdr[kWsTliMagic] == kTliMagic;
  if (!ok && threadIdx.x == 0) raise_status(hdr + kWsStatus, SDV_STATUS_TLI_REUSE);
  return ok;
}

// Four consecutive target ids per thread (one 16-byte inverse load, one
// 16-byte non-temporal store per row) over kRowsPerScatter rows, whose
// gathers are independent and all in flight.  The gathers land anywhere in
// their q rows, so every block of a row group runs on the XCD that owns the
// group (hardware block h runs on XCD h % 8): each row is then fetched into
// one L2 only, where the group's blocks find it.  Needs Vt % 4 == 0 and a
// 16-byte aligned output.
__global__ void __launch_bounds__(256)
q_scatter4_kernel(int64_t rows, int K, int Vt, int nchunks, const float *__restrict__ q,
                  const int *__restrict__ inv, float *__restrict__ out, unsigned *__restrict__ hdr) {
  const int xcd = blockIdx.x % kXcdCount, slot = blockIdx.x / kXcdCount;
  const int64_t group = static_cast<int64_t>(slot / nchunks) * kXcdCount + xcd;
  const int v = ((slot % nchunks) * 256 + static_cast<int>(threadIdx.x)) * 4;
  const int64_t r0 = group * kRowsPerScatter;
  if (v >= Vt || r0 >= rows) return;
  const bool same = map_matches(hdr, K, Vt);
  int4 j = *reinterpret_cast<const int4 *>(inv + v);
  const unsigned uk = same ? static_cast<unsigned>(K) : 0u;     // a foreign map: every entry 0
  j.x = static_cast<unsigned>(j.x) < uk ? j.x : -1;
  j.y = static_cast<unsigned>(j.y) < uk ? j.y : -1;
  j.z = static_cast<unsigned>(j.z) < uk ? j.z : -1;
  j.w = static_cast<unsigned>(j.w) < uk ? j.w : -1;
#pragma unroll
  for (int rr = 0; rr < kRowsPerScatter; ++rr) {
    const int64_t r = r0 + rr;
    if (r >= rows) break;
    const float *qr = q + r * K;
    f32x4v o;
    o.x = j.x >= 0 ? qr[j.x] : 0.0f;
    o.y = j.y >= 0 ? qr[j.y] : 0.0f;
    o.z = j.z >= 0 ? qr[j.z] : 0.0f;
    o.w = j.w >= 0 ? qr[j.w] : 0.0f;
    __builtin_nontemporal_store(o, reinterpret_cast<f32x4v *>(out + r * Vt + v));
  }
}

// Gather form through LDS: one 1024-thread workgroup per (q row, chunk of
// kGatherIds target ids).  Each thread holds 44 of the chunk's target ids
// (eleven runs of four, coalesced) in registers: their inverse entries
// inv[t] (the q column of t, or -1) and their outputs, zero to start.  The q
// row then passes through LDS in slices of at most kQSlice floats (two at K
// = 60000, copied by DMA), and each thread picks up the entries whose column
// falls in the slice; finally the chunk is written with 16-byte
// non-temporal stores.  The chunks of a row run on one XCD (hardware block h
// runs on XCD h % 8), so the row comes from HBM once and from that L2 after.
// (A scatter form that streamed every (target id, q value) pair of the row
// into an LDS chunk of 32768 outputs per workgroup read 480 KB per 128 KB
// written; a gather from L2 moves a 128-byte line per 4-byte entry.)  Needs
// Vt % 4 == 0, K % 4 == 0 and 16-byte aligned q rows and output.
constexpr int kGatherThreads = 1024;
constexpr int kGatherRuns = 11;                                  // runs of four target ids per thread
constexpr int kGatherIds = kGatherThreads * 4 * kGatherRuns;      // 45056 target ids per workgroup
constexpr int kQSlice = 38912;                                   // q floats per LDS slice (152 KB)

__global__ void __launch_bounds__(kGatherThreads)
q_gather_lds_kernel(int64_t rows, int K, int Vt, int nch, int slice, const float *__restrict__ q,
                    const int *__restrict__ inv, float *__restrict__ out, unsigned *__restrict__ hdr) {
  extern __shared__ __attribute__((aligned(16))) float s_q[];
  const int xcd = blockIdx.x % kXcdCount, bslot = blockIdx.x / kXcdCount;
  const int64_t r = static_cast<int64_t>(bslot / nch) * kXcdCount + xcd;
  const int c = bslot % nch;
  if (r >= rows) return;
  const int tid = static_cast<int>(threadIdx.x);
  const int base = c * kGatherIds;
  const bool same = map_matches(hdr, K, Vt);                        // a foreign map: every entry 0
  int4 j[kGatherRuns];
  f32x4v o[kGatherRuns];
#pragma unroll
  for (int g = 0; g < kGatherRuns; ++g) {
    const int t = base + 4 * (tid + g * kGatherThreads);
    j[g] = same && t < Vt ? *reinterpret_cast<const int4 *>(inv + t) : make_int4(-1, -1, -1, -1);
    o[g] = f32x4v{0.0f, 0.0f, 0.0f, 0.0f};
  }
  const float *qr = q + r * K;
  const uint32_t lds_wave = __builtin_amdgcn_readfirstlane(lds_offset(s_q) + (tid / kWave) * kWave * 16);
  for (int lo = 0; same && lo < K; lo += slice) {
    const int len = min(slice, K - lo);                             // a multiple of 4
    // the slice into LDS: float4 i of the slice (lane-contiguous per wave)
    for (int i0 = 0; i0 < len / 4; i0 += kGatherThreads)
      if (i0 + tid < len / 4) dma16(qr + lo + 4 * (i0 + tid), lds_wave + 16u * i0);
    asm volatile("s_waitcnt vmcnt(0)" : : : "memory");              // this wave's copies are in
    __syncthreads();                                                // and everyone's
    const unsigned ulen = static_cast<unsigned>(len);
#pragma unroll
    for (int g = 0; g < kGatherRuns; ++g) {
      if (static_cast<unsigned>(j[g].x - lo) < ulen) o[g].x = s_q[j[g].x - lo];
      if (static_cast<unsigned>(j[g].y - lo) < ulen) o[g].y = s_q[j[g].y - lo];
      if (static_cast<unsigned>(j[g].z - lo) < ulen) o[g].z = s_q[j[g].z - lo];
      if (static_cast<unsigned>(j[g].w - lo) < ulen) o[g].w = s_q[j[g].w - lo];
    }
    __syncthreads();                                                // read before the next slice lands
  }
  float *orow = out + r * Vt;
#pragma unroll
  for (int g = 0; g < kGatherRuns; ++g) {
    const int t = base + 4 * (tid + g * kGatherThreads);
    if (t < Vt) __builtin_nontemporal_store(o[g], reinterpret_cast<f32x4v *>(orow + t));
  }
}

__global__ void q_scatter_kernel(int64_t rows, int K, int Vt, const float *__restrict__ q,
                                 const int *__restrict__ inv, float *__restrict__ out, unsigned *__restrict__ hdr) {
  const int v = blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t r = blockIdx.y;
  if (v >= Vt || r >= rows) return;
  const int j = inv[v];
  const unsigned uk = map_matches(hdr, K, Vt) ? static_cast<unsigned>(K) : 0u;
  out[r * Vt + v] = static_cast<unsigned>(j) < uk ? q[r * K + j] : 0.0f;
}

inline unsigned nblk(int64_t n, int t) { return static_cast<unsigned>((n + t - 1) / t); }

}  // namespace
}  // namespace sdv

using namespace sdv;

extern "C" int32_t sdv_tli_lm_head(int32_t B, int32_t H, int32_t K, const uint16_t *hidden,
                                   const uint16_t *weight, float *logits, void *stream) {
  clear_error();
  SDV_REQUIRE(B >= 0 && H >= 0 && K >= 0, SDV_E_SHAPE, "tli_lm_head: negative size");
  SDV_REQUIRE(H % 32 == 0, SDV_E_UNSUPPORTED, "tli_lm_head: H=%d must be a multiple of 32", H);
  if (B == 0 || K == 0) return SDV_OK;
  SDV_REQUIRE(hidden && weight && logits, SDV_E_NULL, "tli_lm_head: NULL pointer");
  SDV_REQUIRE(reinterpret_cast<uintptr_t>(hidden) % 16 == 0 && reinterpret_cast<uintptr_t>(weight) % 16 == 0,
              SDV_E_SHAPE, "tli_lm_head: hidden and weight must be 16-byte aligned");
  if (H == 0) {
    hipLaunchKernelGGL(fill_i32_kernel, dim3(nblk(static_cast<int64_t>(B) * K, 256)), dim3(256), 0,
                       as_stream(stream), reinterpret_cast<int *>(logits), static_cast<int64_t>(B) * K, 0);
    return check_launch("fill_i32_kernel");
  }
  // hidden rows staged in LDS: one pass of MB 16-row blocks covering B
  const int mb_lds = B <= 16 ? 1 : (B <= 32 ? 2 : 4);
  const size_t lds = static_cast<size_t>(mb_lds) * 16 * (H + kHPad) * 2;
  if (B <= 64 && lds <= static_cast<size_t>(kLdsMax)) {
    auto run = [&](auto kernel, int mb) -> int32_t {
      static thread_local int configured_dev[3] = {-1, -1, -1};
      const int slot = mb == 1 ? 0 : (mb == 2 ? 1 : 2);
      int dev = 0;
      if (hipGetDevice(&dev) != hipSuccess) return fail(SDV_E_HIP, "tli_lm_head: no device");
      if (configured_dev[slot] != dev) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kernel),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, kLdsMax);
        if (e != hipSuccess) return fail(SDV_E_HIP, "tli_lm_head: LDS attribute: %s", hipGetErrorString(e));
        configured_dev[slot] = dev;
      }
      hipLaunchKernelGGL(kernel, dim3(nblk(K, kLdsWaves * 16)), dim3(kLdsWaves * 64), lds, as_stream(stream), B, H, K,
                         hidden, weight, logits);
      return check_launch("lm_head_lds_kernel");
    };
    if (mb_lds == 1) return run(lm_head_lds_kernel<1, kLdsWaves>, 1);
    if (mb_lds == 2) return run(lm_head_lds_kernel<2, kLdsWaves>, 2);
    return run(lm_head_lds_kernel<4, kLdsWaves>, 4);
  }
  const int mpass = kMaxMBlocks * 16;
  dim3 grid(nblk(K, kRowsPerBlock), nblk(B, mpass));
  if (B <= 16) {
    hipLaunchKernelGGL((lm_head_kernel<1, kNBlocks>), grid, dim3(kGemmThreads), 0, as_stream(stream), B, H, K, hidden,
                       weight, logits);
  } else if (B <= 32) {
    hipLaunchKernelGGL((lm_head_kernel<2, kNBlocks>), grid, dim3(kGemmThreads), 0, as_stream(stream), B, H, K, hidden,
                       weight, logits);
  } else if (B <= 64) {
    hipLaunchKernelGGL((lm_head_kernel<4, kNBlocks>), grid, dim3(kGemmThreads), 0, as_stream(stream), B, H, K, hidden,
                       weight, logits);
  } else {
    hipLaunchKernelGGL((lm_head_kernel<kMaxMBlocks, kNBlocks>), grid, dim3(kGemmThreads), 0, as_stream(stream), B, H, K,
                       hidden, weight, logits);
  }
  return check_launch("lm_head_kernel");
}

extern "C" int32_t sdv_tli_build_maps(int32_t K, const int32_t *inter_ids, const int32_t *tgt_ids,
                                      int32_t V_draft, int32_t V_target, int32_t fallback, int32_t *d2t,
                                      int32_t *t2d, void *stream) {
  clear_error();
  SDV_REQUIRE(K >= 0 && V_draft >= 1 && V_target >= 1, SDV_E_SHAPE, "tli_build_maps: bad sizes");
  SDV_REQUIRE(d2t && t2d && (K == 0 || (inter_ids && tgt_ids)), SDV_E_NULL, "tli_build_maps: NULL pointer");
  hipStream_t st = as_stream(stream);
  hipLaunchKernelGGL(fill_i32_kernel, dim3(nblk(V_draft, 256)), dim3(256), 0, st, d2t,
                     static_cast<int64_t>(V_draft), -1);
  hipLaunchKernelGGL(fill_i32_kernel, dim3(nblk(V_target, 256)), dim3(256), 0, st, t2d,
                     static_cast<int64_t>(V_target), fallback);
  if (K > 0)
    hipLaunchKernelGGL(scatter_maps_kernel, dim3(nblk(K, 256)), dim3(256), 0, st, K, inter_ids, tgt_ids,
                       V_draft, V_target, d2t, t2d);
  return check_launch("tli_build_maps");
}

extern "C" int32_t sdv_tli_map_ids(const int32_t *table, int32_t table_len, const int32_t *ids, int64_t n,
                                   int32_t *out, void *stream) {
  clear_error();
  SDV_REQUIRE(n >= 0 && table_len >= 0, SDV_E_SHAPE, "tli_map_ids: negative size");
  if (n == 0) return SDV_OK;
  SDV_REQUIRE(table && ids && out, SDV_E_NULL, "tli_map_ids: NULL pointer");
  hipLaunchKernelGGL(map_ids_kernel, dim3(nblk(n, 256)), dim3(256), 0, as_stream(stream), table, table_len, ids,
                     n, out);
  return check_launch("map_ids_kernel");
}

extern "C" int32_t sdv_tli_constrain_draft_logits(int32_t B, int32_t K, int32_t V_draft, const float *pruned,
                                                  const int32_t *inter_ids, float *full, void *stream) {
  clear_error();
  SDV_REQUIRE(B >= 0 && K >= 0 && V_draft >= 1 && K <= V_draft, SDV_E_SHAPE, "tli_constrain: bad sizes");
  if (B == 0) return SDV_OK;
  SDV_REQUIRE(full && (K == 0 || (pruned && inter_ids)), SDV_E_NULL, "tli_constrain: NULL pointer");
  if (V_draft % 4 == 0 && reinterpret_cast<uintptr_t>(full) % 16 == 0) {
    hipLaunchKernelGGL(constrain4_kernel, dim3(nblk(V_draft / 4, 256), nblk(B, kRowsPerScatter)), dim3(256), 0,
                       as_stream(stream), B, K, V_draft, pruned, inter_ids, full);
    return check_launch("constrain4_kernel");
  }
  hipLaunchKernelGGL(constrain_kernel, dim3(nblk(V_draft, 256)), dim3(256), 0, as_stream(stream), B, K, V_draft,
                     pruned, inter_ids, full);
  return check_launch("constrain_kernel");
}

// Workspace: the header (status, and the K and V_target of the map), then
// the inverse of tgt_ids [V_target].
extern "C" size_t sdv_tli_q_scatter_workspace_size(int32_t V_target) {
  return V_target > 0 ? kWsHeaderBytes + align_up(static_cast<size_t>(V_target) * sizeof(int), 256) : 0;
}

extern "C" int32_t sdv_tli_q_scatter(int64_t rows, int32_t K, int32_t V_target, const float *q_pruned,
                                     const int32_t *tgt_ids, float *q_target, void *ws, size_t ws_bytes,
                                     void *stream) {
  clear_error();
  SDV_REQUIRE(rows >= 0 && K >= 0 && V_target >= 1 && K <= V_target, SDV_E_SHAPE, "tli_q_scatter: bad sizes");
  SDV_REQUIRE(rows <= 65535, SDV_E_UNSUPPORTED, "tli_q_scatter: rows above 65535");
  if (rows == 0) return SDV_OK;
  SDV_REQUIRE(q_target && (K == 0 || q_pruned), SDV_E_NULL, "tli_q_scatter: NULL pointer");
  if (K == 0) {                          // nothing to scatter: zeros, the workspace untouched
    const int64_t n = rows * static_cast<int64_t>(V_target);
    SDV_REQUIRE((n + 255) / 256 < (1LL << 31), SDV_E_UNSUPPORTED, "tli_q_scatter: output too large");
    hipLaunchKernelGGL(fill_i32_kernel, dim3(nblk(n, 256)), dim3(256), 0, as_stream(stream),
                       reinterpret_cast<int *>(q_target), n, 0);
    return check_launch("fill_i32_kernel");
  }
  const size_t need = sdv_tli_q_scatter_workspace_size(V_target);
  SDV_REQUIRE(ws && ws_bytes >= need, SDV_E_WORKSPACE, "tli_q_scatter: workspace of %zu bytes needed", need);
  unsigned *hdr = ws_header(ws);
  int *inv = reinterpret_cast<int *>(static_cast<char *>(ws) + kWsHeaderBytes);
  hipStream_t st = as_stream(stream);
  if (tgt_ids) {                         // else: the inverse an earlier call left in ws
    hipLaunchKernelGGL(fill_i32_kernel, dim3(nblk(V_target, 256)), dim3(256), 0, st, inv,
                       static_cast<int64_t>(V_target), -1);
    hipLaunchKernelGGL(inverse_kernel, dim3(K > 0 ? nblk(K, 256) : 1), dim3(256), 0, st, K, tgt_ids, V_target, inv,
                       hdr);
  }
  if (V_target % 4 == 0 && K % 4 == 0 && reinterpret_cast<uintptr_t>(q_target) % 16 == 0 &&
      reinterpret_cast<uintptr_t>(q_pruned) % 16 == 0) {
    // slices of at most kQSlice floats, equal up to the last, multiples of 4
    const int nslices = K > 0 ? (K + kQSlice - 1) / kQSlice : 1;
    const int slice = static_cast<int>(align_up(static_cast<size_t>((K + nslices - 1) / nslices), 4));
    const size_t lds = static_cast<size_t>(std::max(slice, 4)) * sizeof(float);
    static thread_local int configured_dev = -1;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(SDV_E_HIP, "tli_q_scatter: no device");
    if (configured_dev != dev) {
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(q_gather_lds_kernel),
                                         hipFuncAttributeMaxDynamicSharedMemorySize,
                                         static_cast<int>(kQSlice * sizeof(float)));
      if (e != hipSuccess) return fail(SDV_E_HIP, "tli_q_scatter: LDS attribute: %s", hipGetErrorString(e));
      configured_dev = dev;
    }
    const int nch = static_cast<int>(nblk(V_target, kGatherIds));
    const int64_t per_xcd = (rows + kXcdCount - 1) / kXcdCount;       // rows per XCD
    const int64_t blocks = per_xcd * nch * kXcdCount;
    SDV_REQUIRE(blocks < (1LL << 31), SDV_E_UNSUPPORTED, "tli_q_scatter: grid too large");
    hipLaunchKernelGGL(q_gather_lds_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kGatherThreads), lds, st,
                       rows, K, V_target, nch, std::max(slice, 4), q_pruned, inv, q_target, hdr);
    return check_launch("q_gather_lds_kernel");
  }
  if (V_target % 4 == 0 && reinterpret_cast<uintptr_t>(q_target) % 16 == 0) {
    const int nchunks = static_cast<int>(nblk(V_target / 4, 256));
    const int64_t groups = nblk(rows, kRowsPerScatter);
    const int64_t per_xcd = (groups + kXcdCount - 1) / kXcdCount;     // row groups per XCD
    hipLaunchKernelGGL(q_scatter4_kernel, dim3(static_cast<unsigned>(per_xcd * nchunks * kXcdCount)), dim3(256), 0,
                       st, rows, K, V_target, nchunks, q_pruned, inv, q_target, hdr);
    return check_launch("q_scatter4_kernel");
  }
  hipLaunchKernelGGL(q_scatter_kernel, dim3(nblk(V_target, 256), static_cast<unsigned>(rows)), dim3(256), 0, st,
                     rows, K, V_target, q_pruned, inv, q_target, hdr);
  return check_launch("q_scatter_kernel");
}
