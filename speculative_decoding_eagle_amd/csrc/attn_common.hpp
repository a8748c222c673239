// Pieces shared by the two tree-verify attention kernels (attn.hip: units of
// up to 128 query rows; attn_wide.hip: wider units, keys split over
// workgroups): fragment types, the LDS chunk swizzle, the LDS-DMA issue,
// cross-lane reductions and the in-kernel longest-first request ranking.
#pragma once

#include <cmath>

#include "common.hpp"

namespace sdv {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

constexpr int kAttnThreads = 512;   // eight waves per workgroup (both kernels)
constexpr int kTile = 64;           // key positions per tile
constexpr int kStages = 4;          // tiles per LDS ring (one ring for K, one for V)
constexpr int kXcds = 8;
constexpr int kPageCache = 4096;    // page-table entries cached in LDS
constexpr int kRankMax = 1024;      // requests ranked in-kernel; larger batches keep their order

// Per head dimension: bytes and 16-byte chunks of a key row, and how the
// eight waves split one tile's DMA (wave w moves key rows 8w .. 8w+7).
template <int D>
struct KvTile {
  static constexpr int ROW = 2 * D;                       // bytes per key row
  static constexpr int CHUNKS = D / 8;                    // 16-byte chunks per row
  static constexpr int KPI = 64 / CHUNKS;                 // key rows per DMA instruction (1 KB)
  static constexpr int IPW = 8 / KPI;                     // DMA instructions per wave per tile and tensor
  static constexpr int DS = D / 32;                       // k-steps of QK^T
  static constexpr int NO = D / 16;                       // 16-wide d blocks of O^T per row block
  static constexpr int TILE_BYTES = kTile * ROW;
  static constexpr int RINGS = 2 * kStages * TILE_BYTES;  // K ring, then V ring
};

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40);   // NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Chunk swizzle of key row r (depends on r % 16 only), for two LDS read
// patterns.  K fragments (16-byte reads): the 16 rows read by one
// quarter-wave map a fixed chunk to 16 distinct bank groups.  V^T
// (transposing 8-byte reads): a half-wave reads chunk pair (2db, 2db+1) of
// rows 0..7 (or 8..15), and swz(r) / 2 differs across those rows, so the 16
// chunk reads hit distinct bank groups.  (A 256-byte row covers all 64
// banks: the bank group is the chunk; a 128-byte row covers half, so for
// D = 64 rows of either parity are told apart separately.)
template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D == 128) {
    return ((r & 7) << 1) | ((r >> 3) & 1);
  } else {
    return (r & 6) | ((r >> 3) & 1);
  }
}

// 4 bytes per lane from global memory straight into LDS (lane L writes LDS
// bytes lds_addr + 4*L .. +3); same conventions as dma16.
__device__ __forceinline__ void dma4(const void *gaddr, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" : : "v"(gaddr), "s"(lds_addr) : "memory", "m0");
}

// Lane l's value combined with lane l^16's (l^32's): the row-half swap
// instructions hand every lane the pair {x[l], x[l^16]} ({x[l], x[l^32]}).
__device__ __forceinline__ float max_xor16(float x) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return vmax(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return vmax(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float sum_xor16(float x) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float sum_xor32(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

namespace {
// Source of the DMA for key positions outside the request: 256 zero bytes,
// never written.
__device__ __attribute__((aligned(256))) uint16_t g_zero16[128];
}  // namespace

// The request of rank r when requests are ranked by prefix length (longest
// first, then lower index).  Every block ranks the (small) batch itself from
// an LDS copy of the prefix lengths; s_len is LDS scratch of B ints.
__device__ __forceinline__ int request_of_rank(int r, int B, const int *__restrict__ prefix_len, int *s_len,
                                               int *s_pick) {
  if (B > kRankMax) return r;
  const int tid = threadIdx.x;
  for (int i = tid; i < B; i += kAttnThreads) s_len[i] = prefix_len[i];
  __syncthreads();
  for (int c = tid; c < B; c += kAttnThreads) {
    const int Lc = s_len[c];
    int rk = 0;
    for (int o = 0; o < B; ++o) {
      const int Lo = s_len[o];
      rk += (Lo > Lc) | ((Lo == Lc) & (o < c));
    }
    if (rk == r) *s_pick = c;
  }
  __syncthreads();
  return *s_pick;
}

// The wide kernel's workspace: the status header, a fixed region of
// counters (two per unit) that every call leaves at zero, whatever the shape,
// then two partial-result slots per workgroup of the persistent schedule.
constexpr int kAttnSyncWords = 8192;

// Workspace of the wide kernel's persistent schedule for `units` (request,
// KV head, row block) units; 0 when it is not offered (more than
// kAttnSyncWords / 2 units).
size_t attn_wide_workspace(int64_t units, int D);

// Launches the wide kernel (query rows per unit above 128).  split: run the
// persistent schedule (every compute unit streams an equal share of all
// units' key tiles; units cut between workgroups merge their partial
// softmax states), which needs ws: attn_wide_workspace bytes, zero-filled
// before first use (calls leave the counters at zero).  Otherwise one
// workgroup per (unit, row block).
int32_t launch_attn_wide(hipStream_t st, const sdv_attn_shape &sh, int pshift, float scale_log2, int nrb, bool split,
                         const uint16_t *q, const uint16_t *k_pool, const uint16_t *v_pool,
                         const int32_t *page_table, const int32_t *prefix_len, const uint32_t *mask_bits,
                         uint16_t *out, float *lse, void *ws);

}  // namespace sdv
