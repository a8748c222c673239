// A5: tree-verify attention -- one target pass over the prefix plus the
// candidate tree with the tree mask ("EAGLE speculative decoding in four
// parts", "Self-test" answer 1, "Exercises" question 1 and "Design
// trade-offs"; "[SGLang] Multi-Layer EAGLE" section 6, TARGET_VERIFY).
//
// Layout of the work.  GQA packs the Hq/Hkv query heads that share a KV head
// with the N tree nodes into N*G query rows (row = node*G + g).  A block of
// four waves owns 64 of those rows of one (request, KV head) and streams the
// request's keys in tiles of 64 positions through LDS:
//   * K tile [64 keys][D] (row-padded) and V tile transposed to [D][64 keys],
//     gathered through the page table (page size 1: a slot map);
//   * wave w takes keys 16w..16w+15 of every tile for all 64 rows (the
//     waves split the key axis, so each K/V byte is read from LDS once);
//   * S^T = K Q^T with bf16 MFMA 16x16x32 (Q fragments stay in registers),
//     online softmax in fp32 with exp2, O^T += V^T P^T with MFMA 16x16x16,
//     so every lane keeps the statistics of its own query row;
//   * at the end the four waves' (max, sum, O) are merged through LDS in a
//     fixed order (deterministic) and written as bf16.
// Row blocks of one (request, KV head) are placed on one XCD (the dispatcher
// deals blocks round-robin over the 8 XCDs) so they share that XCD's L2.
#include <cmath>

#include "common.hpp"

namespace sdv {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

constexpr int kAttnThreads = 256;
constexpr int kRows = 64;          // query rows per block
constexpr int kTile = 64;          // key positions per tile
constexpr int kXcds = 8;

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40);   // NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

template <int D>
struct AttnSmem {
  static constexpr int kKStride = D + 8;          // bf16 elements per K row (16-byte pad)
  static constexpr int kVStride = kTile + 8;      // bf16 elements per transposed V row
  static constexpr int kKBytes = kTile * kKStride * 2;
  static constexpr int kVBytes = D * kVStride * 2;
  static constexpr int kMergeBytes = 2 * kRows * D * 4;   // two fp32 O tiles
  static constexpr int kBytes = (kKBytes + kVBytes) > kMergeBytes ? (kKBytes + kVBytes) : kMergeBytes;
};

template <int D>
__global__ void __launch_bounds__(kAttnThreads, 2)
tree_attn_kernel(int B, int N, int Hq, int Hkv, int page, int max_pages, int64_t num_slots, float scale_log2,
                 int nrb, int units_total, const uint16_t *__restrict__ q, const uint16_t *__restrict__ kpool,
                 const uint16_t *__restrict__ vpool, const int *__restrict__ table,
                 const int *__restrict__ prefix_len, const uint32_t *__restrict__ mask_bits,
                 uint16_t *__restrict__ out, float *__restrict__ lse) {
  using Sm = AttnSmem<D>;
  constexpr int DS = D / 32;        // k-steps of the QK^T contraction
  constexpr int DB = D / 16;        // 16-wide d blocks of the output
  constexpr int RB = kRows / 16;    // 16-row blocks per wave
  __shared__ __attribute__((aligned(16))) unsigned char smem[Sm::kBytes];
  __shared__ float s_m[4][kRows];
  __shared__ float s_l[4][kRows];
  __shared__ uint32_t s_mask[kRows / 1][8];

  // XCD-aware placement: blocks x, x+8, x+16, ... run on one XCD; give them
  // consecutive logical indices so the row blocks of a unit share an L2.
  const int nblocks = gridDim.x;
  const int per_xcd = nblocks / kXcds;
  const int logical = (blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
  if (logical >= units_total * nrb) return;
  const int unit = logical / nrb;
  const int rblk = logical % nrb;
  const int b = unit / Hkv;
  const int kvh = unit % Hkv;
  const int G = Hq / Hkv;
  const int W = (N + 31) / 32;

  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int l = lane_id();
  const int l16 = l & 15;
  const int g4 = l >> 4;

  const int L = prefix_len[b];
  const int total_keys = L + N;
  const int *trow = table + static_cast<int64_t>(b) * max_pages;
  const bool req_ok = L >= 0 && static_cast<int64_t>(total_keys) <= static_cast<int64_t>(max_pages) * page;

  // tree mask rows of the nodes this block covers
  const int row0 = rblk * kRows;
  const int node0 = row0 / G;
  const int nodes_here = min(N - node0, (kRows + G - 1) / G + 1);
  for (int x = tid; x < kRows * 8; x += kAttnThreads) {
    const int nn = x / 8, w = x % 8;
    uint32_t v = 0;
    if (nn < nodes_here && w < W) v = mask_bits[(static_cast<int64_t>(b) * N + node0 + nn) * W + w];
    s_mask[nn][w] = v;
  }

  // Q fragments (B operand of S^T = K Q^T): lane holds Q[row][8*g4 .. +7] of k-step ds
  bf16x8 qf[RB][DS];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int r = row0 + rb * 16 + l16;
    const int node = r / G, g = r % G;
    const bool ok = node < N;
    const uint16_t *qp = q + ((static_cast<int64_t>(b) * N + (ok ? node : 0)) * Hq + kvh * G + g) * D;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      uint4 u = ok ? *reinterpret_cast<const uint4 *>(qp + ds * 32 + 8 * g4) : make_uint4(0, 0, 0, 0);
      __builtin_memcpy(&qf[rb][ds], &u, 16);
    }
  }

  f32x4 o[RB][DB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int db = 0; db < DB; ++db) o[rb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[RB], l_run[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m_run[rb] = -INFINITY;
    l_run[rb] = 0.f;
  }

  uint16_t *k_lds = reinterpret_cast<uint16_t *>(smem);
  uint16_t *v_lds = reinterpret_cast<uint16_t *>(smem + Sm::kKBytes);
  const int chunks_per_key = D / 8;

  const int ntiles = req_ok ? (total_keys + kTile - 1) / kTile : 0;
  for (int tile = 0; tile < ntiles; ++tile) {
    const int pos0 = tile * kTile;
    __syncthreads();
    // ---- K tile: 16-byte chunks, consecutive lanes along one key row
    for (int c = tid; c < kTile * chunks_per_key; c += kAttnThreads) {
      const int kk = c / chunks_per_key, col = c % chunks_per_key;
      const int pos = pos0 + kk;
      uint4 u = make_uint4(0, 0, 0, 0);
      if (pos < total_keys) {
        const int64_t slot = static_cast<int64_t>(trow[pos / page]) * page + pos % page;
        if (slot >= 0 && slot < num_slots)
          u = *reinterpret_cast<const uint4 *>(kpool + (slot * Hkv + kvh) * D + col * 8);
      }
      *reinterpret_cast<uint4 *>(k_lds + kk * Sm::kKStride + col * 8) = u;
    }
    // ---- V tile, transposed: a thread takes two adjacent keys of one 8-wide d chunk
    for (int c = tid; c < (kTile / 2) * chunks_per_key; c += kAttnThreads) {
      const int kp = c % (kTile / 2), col = c / (kTile / 2);
      uint4 u[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int pos = pos0 + 2 * kp + h;
        u[h] = make_uint4(0, 0, 0, 0);
        if (pos < total_keys) {
          const int64_t slot = static_cast<int64_t>(trow[pos / page]) * page + pos % page;
          if (slot >= 0 && slot < num_slots)
            u[h] = *reinterpret_cast<const uint4 *>(vpool + (slot * Hkv + kvh) * D + col * 8);
        }
      }
      const uint16_t *e0 = reinterpret_cast<const uint16_t *>(&u[0]);
      const uint16_t *e1 = reinterpret_cast<const uint16_t *>(&u[1]);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t pair = static_cast<uint32_t>(e0[j]) | (static_cast<uint32_t>(e1[j]) << 16);
        *reinterpret_cast<uint32_t *>(v_lds + (col * 8 + j) * Sm::kVStride + 2 * kp) = pair;
      }
    }
    __syncthreads();

    // ---- S^T for this wave's 16 keys: A = K[key][d] from LDS, B = Q^T
    const int key_base = wave * 16;
    f32x4 s[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) s[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      bf16x8 kf;
      __builtin_memcpy(&kf, k_lds + (key_base + l16) * Sm::kKStride + ds * 32 + 8 * g4, 16);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) s[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[rb][ds], s[rb], 0, 0, 0);
    }

    // ---- mask, online softmax (lane: row l16 of each row block; keys 4*g4+i)
    s16x4 pf[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int r = row0 + rb * 16 + l16;
      const int nn = r / G - node0;
      float v[4];
      float tmax = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int pos = pos0 + key_base + 4 * g4 + i;
        bool vis = pos < L;
        if (!vis && pos < total_keys) {
          const int j = pos - L;
          vis = (nn >= 0 && nn < kRows) && ((s_mask[nn][j >> 5] >> (j & 31)) & 1u);
        }
        v[i] = vis ? s[rb][i] * scale_log2 : -INFINITY;
        tmax = fmaxf(tmax, v[i]);
      }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16, kWave));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32, kWave));
      const float m_new = fmaxf(m_run[rb], tmax);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = exp2f(m_run[rb] - m_use);
      m_run[rb] = m_new;
      float psum = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = exp2f(v[i] - m_use);
        psum += p;
        pf[rb][i] = static_cast<short>(f32_to_bf16_rne(p));
      }
      l_run[rb] = l_run[rb] * alpha + psum;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        o[rb][db][0] *= alpha;
        o[rb][db][1] *= alpha;
        o[rb][db][2] *= alpha;
        o[rb][db][3] *= alpha;
      }
    }

    // ---- O^T += V^T P^T: A = V^T[d][keys 4*g4..+3] (LDS), B = P^T (registers)
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      s16x4 vf;
      __builtin_memcpy(&vf, v_lds + (db * 16 + l16) * Sm::kVStride + key_base + 4 * g4, 8);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) o[rb][db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vf, pf[rb], o[rb][db], 0, 0, 0);
    }
  }

  // ---- merge the four waves (fixed order) and write
  __syncthreads();
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    float lt = l_run[rb];
    lt += __shfl_xor(lt, 16, kWave);
    lt += __shfl_xor(lt, 32, kWave);
    if (g4 == 0) {
      s_m[wave][rb * 16 + l16] = m_run[rb];
      s_l[wave][rb * 16 + l16] = lt;
    }
  }
  __syncthreads();
  float fac[RB];
  float mrow[RB], lrow[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int r = rb * 16 + l16;
    float M = -INFINITY;
    for (int w = 0; w < 4; ++w) M = fmaxf(M, s_m[w][r]);
    const float Mu = M == -INFINITY ? 0.f : M;
    float Lsum = 0.f;
    for (int w = 0; w < 4; ++w) Lsum += s_l[w][r] * exp2f(s_m[w][r] - Mu);
    fac[rb] = Lsum > 0.f ? exp2f(m_run[rb] - Mu) / Lsum : 0.f;
    mrow[rb] = Mu;
    lrow[rb] = Lsum;
  }
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) o[rb][db][i] *= fac[rb];

  // O^T fragment: lane holds d = db*16 + 4*g4 + i of row rb*16 + l16
  float *mbuf = reinterpret_cast<float *>(smem);            // two [kRows][D] fp32 tiles
  auto put = [&](int which) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          mbuf[(which * kRows + rb * 16 + l16) * D + db * 16 + 4 * g4 + i] = o[rb][db][i];
  };
  auto add = [&](int which) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          o[rb][db][i] += mbuf[(which * kRows + rb * 16 + l16) * D + db * 16 + 4 * g4 + i];
  };
  if (wave >= 2) put(wave - 2);
  __syncthreads();
  if (wave < 2) add(wave);
  __syncthreads();
  if (wave == 1) put(0);
  __syncthreads();
  if (wave == 0) {
    add(0);
    put(0);
  }
  __syncthreads();
  // coalesced bf16 store of the 64 x D tile: 8 values (16 bytes) per item
  for (int x = tid; x < kRows * (D / 8); x += kAttnThreads) {
    const int r = x / (D / 8), c8 = x % (D / 8);
    const int gr = row0 + r;
    const int node = gr / G, g = gr % G;
    if (node >= N) continue;
    uint16_t h[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) h[j] = f32_to_bf16_rne(mbuf[r * D + c8 * 8 + j]);
    uint4 u;
    __builtin_memcpy(&u, h, 16);
    *reinterpret_cast<uint4 *>(out + ((static_cast<int64_t>(b) * N + node) * Hq + kvh * G + g) * D + c8 * 8) = u;
  }
  if (lse && wave == 0 && g4 == 0) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int gr = row0 + rb * 16 + l16;
      const int node = gr / G, g = gr % G;
      if (node < N)
        lse[(static_cast<int64_t>(b) * N + node) * Hq + kvh * G + g] =
            lrow[rb] > 0.f ? (mrow[rb] + log2f(lrow[rb])) * 0.69314718055994531f : -INFINITY;
    }
  }
}

}  // namespace
}  // namespace sdv

using namespace sdv;

extern "C" size_t sdv_tree_verify_attention_workspace_size(sdv_attn_shape) { return 0; }

extern "C" int32_t sdv_tree_verify_attention(sdv_attn_shape sh, float sm_scale, const uint16_t *q,
                                             const uint16_t *k_pool, const uint16_t *v_pool,
                                             const int32_t *page_table, const int32_t *prefix_len,
                                             const uint32_t *mask_bits, uint16_t *out, float *lse, void *ws,
                                             size_t ws_bytes, void *stream) {
  (void)ws;
  (void)ws_bytes;
  clear_error();
  SDV_REQUIRE(sh.B >= 0 && sh.N >= 1 && sh.Hq >= 1 && sh.Hkv >= 1 && sh.page >= 1 && sh.max_pages >= 1 &&
                  sh.num_slots >= 0,
              SDV_E_SHAPE, "tree_verify_attention: bad sizes");
  SDV_REQUIRE(sh.Hq % sh.Hkv == 0, SDV_E_SHAPE, "tree_verify_attention: Hq %% Hkv != 0");
  SDV_REQUIRE(sh.D == 64 || sh.D == 128, SDV_E_UNSUPPORTED, "tree_verify_attention: D=%d not in {64,128}", sh.D);
  SDV_REQUIRE(sh.N <= 256 && sh.Hq / sh.Hkv <= 16, SDV_E_UNSUPPORTED,
              "tree_verify_attention: N <= 256 and Hq/Hkv <= 16 required");
  if (sh.B == 0) return SDV_OK;
  SDV_REQUIRE(q && k_pool && v_pool && page_table && prefix_len && mask_bits && out, SDV_E_NULL,
              "tree_verify_attention: NULL pointer");
  SDV_REQUIRE(reinterpret_cast<uintptr_t>(q) % 16 == 0 && reinterpret_cast<uintptr_t>(k_pool) % 16 == 0 &&
                  reinterpret_cast<uintptr_t>(v_pool) % 16 == 0 && reinterpret_cast<uintptr_t>(out) % 16 == 0,
              SDV_E_SHAPE, "tree_verify_attention: q, pools and out must be 16-byte aligned");
  const int G = sh.Hq / sh.Hkv;
  const int nrb = (sh.N * G + kRows - 1) / kRows;
  const int units = sh.B * sh.Hkv;
  int64_t blocks = static_cast<int64_t>(units) * nrb;
  blocks = (blocks + kXcds - 1) / kXcds * kXcds;
  SDV_REQUIRE(blocks < (1LL << 31), SDV_E_UNSUPPORTED, "tree_verify_attention: grid too large");
  const float scale = sm_scale > 0.f ? sm_scale : 1.0f / sqrtf(static_cast<float>(sh.D));
  const float scale_log2 = scale * 1.4426950408889634f;
  hipStream_t st = as_stream(stream);
  if (sh.D == 64)
    hipLaunchKernelGGL(tree_attn_kernel<64>, dim3(static_cast<unsigned>(blocks)), dim3(kAttnThreads), 0, st, sh.B,
                       sh.N, sh.Hq, sh.Hkv, sh.page, sh.max_pages, sh.num_slots, scale_log2, nrb, units, q, k_pool,
                       v_pool, page_table, prefix_len, mask_bits, out, lse);
  else
    hipLaunchKernelGGL(tree_attn_kernel<128>, dim3(static_cast<unsigned>(blocks)), dim3(kAttnThreads), 0, st, sh.B,
                       sh.N, sh.Hq, sh.Hkv, sh.page, sh.max_pages, sh.num_slots, scale_log2, nrb, units, q, k_pool,
                       v_pool, page_table, prefix_len, mask_bits, out, lse);
  return check_launch("tree_attn_kernel");
}
