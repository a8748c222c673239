// A5: tree-verify attention -- one target pass over the prefix plus the
// candidate tree with the tree mask ("EAGLE speculative decoding in four
// parts", "Self-test" answer 1, "Exercises" question 1 and "Design
// trade-offs"; "[SGLang] Multi-Layer EAGLE" section 6, TARGET_VERIFY).
//
// Work layout.  GQA packs the G = Hq/Hkv query heads that share a KV head
// with the N tree nodes into N*G query rows (row = node*G + g).  A block of
// eight waves owns 128 of those rows of one (request, KV head) and streams
// the request's keys in tiles of 64 positions.  Wave (rh, kh) computes rows
// 32*rh .. +31 against keys 32*kh .. +31 of every tile, so each wave holds a
// 32 x D fp32 accumulator and two row blocks of Q fragments in registers.
//   * K and V tiles go from the paged pool straight into LDS with
//     global_load_lds_dwordx4 (16 bytes per lane, a wave fills 1 KB per
//     instruction) through a ring of four K tiles and a ring of four V
//     tiles, the K stream one tile ahead (the scores of tile t+1 are computed
//     while tile t's softmax runs): every tile's K and V get three steps to
//     arrive.  No registers stage the data.
//   * LDS rows are unpadded; 16-byte chunks are XOR-swizzled per row so that
//     the MFMA fragment reads below hit distinct banks.
//   * S^T = K Q^T and O^T += V^T P^T on bf16 MFMA 16x16x32; each V^T
//     operand is two transposing LDS reads (ds_read_b64_tr_b16), P is
//     rounded to bf16.  The scores of tile t+1 are issued interleaved with
//     the exponentials of tile t (a fixed issue order).
//   * Every lane keeps the softmax state of its own query row; scores are
//     scaled into log2 units and exponentiated with exp2; the reference max
//     moves only when a score exceeds it by more than 2^8, so the O rescale
//     is rare.  Row maxima and sums cross lanes with the row-half swap
//     instructions, not LDS permutes.
//   * Page ids come from an LDS copy of the request's page-table row,
//     refreshed once per window of kPageCache pages.
//   * The two key-half waves of a row quarter are merged through LDS in a
//     fixed order (deterministic) and the 128 x D tile is stored as bf16.
// Scheduling: each block ranks the requests by prefix length (longest
// first) and takes its unit by rank; blocks are dealt round-robin over the 8 XCDs, so units are
// interleaved over XCDs in that order while the row blocks of one unit stay
// on one XCD and share its L2.
#include <type_traits>

#include "attn_common.hpp"

namespace sdv {
namespace {

constexpr int kRows = 128;          // query rows per block

template <int D>
struct AttnCfg : KvTile<D> {
  static constexpr int SMEM = KvTile<D>::RINGS;           // K ring, V ring; also holds the fp32 merge buffer
  static_assert(kRows * D * 4 <= SMEM, "merge buffer must fit");
};

template <int D>
__global__ void __launch_bounds__(kAttnThreads, 2)
tree_attn_kernel(int B, int N, int Hq, int Hkv, int pshift, int max_pages, int64_t num_slots, float scale_log2,
                 int nrb, const uint16_t *__restrict__ q, const uint16_t *__restrict__ kpool,
                 const uint16_t *__restrict__ vpool, const int *__restrict__ table,
                 const int *__restrict__ prefix_len, const uint32_t *__restrict__ mask_bits,
                 uint16_t *__restrict__ out, float *__restrict__ lse) {
  using C = AttnCfg<D>;
  constexpr int RB = 2;                       // 16-row blocks per wave
  constexpr int KB = 2;                       // 16-key blocks per wave per tile
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  __shared__ float s_m[2][kRows];
  __shared__ float s_l[2][kRows];
  __shared__ uint32_t s_mask[kRows][8];
  __shared__ int s_page[kPageCache];
  __shared__ int s_pick;

  // hardware block h runs on XCD h % 8 as that XCD's (h / 8)-th block
  const int xcd = blockIdx.x % kXcds;
  const int slot_in_xcd = blockIdx.x / kXcds;
  const int rank = (slot_in_xcd / nrb) * kXcds + xcd;       // unit rank, longest requests first
  const int rblk = slot_in_xcd % nrb;
  if (rank >= B * Hkv) return;
  const int b = request_of_rank(rank / Hkv, B, prefix_len, reinterpret_cast<int *>(smem), &s_pick);
  const int kvh = rank % Hkv;
  const int G = Hq / Hkv;
  const int W = (N + 31) / 32;
  const int pmask = (1 << pshift) - 1;

  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int rh = wave >> 1, kh = wave & 1;    // rows 32*rh .. +31, keys 32*kh .. +31
  const int l = lane_id();
  const int l16 = l & 15;
  const int g4 = l >> 4;

  // the ranking left the batch's prefix lengths in LDS (one global read fewer on the way to the first tile)
  const int L = B <= kRankMax ? reinterpret_cast<const int *>(smem)[b] : prefix_len[b];
  const int total = L + N;
  const int *trow = table + static_cast<int64_t>(b) * max_pages;
  const bool req_ok = L >= 0 && static_cast<int64_t>(total) <= (static_cast<int64_t>(max_pages) << pshift);
  const int ntiles = req_ok ? (total + kTile - 1) / kTile : 0;
  const int total_pages = req_ok ? (total + pmask) >> pshift : 0;   // page-table entries the request owns
  const int win_tiles = pshift >= 19 ? (1 << 30) : (kPageCache << pshift) / kTile;   // tiles per page window

  const int row0 = rblk * kRows;
  const int node0 = row0 / G;
  for (int x = tid; x < kRows * 8; x += kAttnThreads) {
    const int nn = x / 8, w = x % 8;
    uint32_t v = 0;
    if (node0 + nn < N && w < W) v = mask_bits[(static_cast<int64_t>(b) * N + node0 + nn) * W + w];
    s_mask[nn][w] = v;
  }

  // this lane's rows: row0 + 32*rh + 16*rb + l16
  int nrel[RB];
  bf16x8 qf[RB][C::DS];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int r = row0 + 32 * rh + 16 * rb + l16;
    const int node = r / G, g = r % G;
    nrel[rb] = node - node0;
    const bool ok = node < N;
    const uint16_t *qp = q + ((static_cast<int64_t>(b) * N + (ok ? node : 0)) * Hq + kvh * G + g) * D;
#pragma unroll
    for (int ds = 0; ds < C::DS; ++ds) {
      uint4 u = ok ? *reinterpret_cast<const uint4 *>(qp + ds * 32 + 8 * g4) : make_uint4(0, 0, 0, 0);
      __builtin_memcpy(&qf[rb][ds], &u, 16);
    }
  }
  f32x4 o[RB][C::NO];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int j = 0; j < C::NO; ++j) o[rb][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[RB], l_run[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m_run[rb] = -INFINITY;
    l_run[rb] = 0.f;
  }

  auto refresh_pages = [&](int first_tile) {
    const int p0 = (first_tile * kTile) >> pshift;
    for (int x = tid; x < kPageCache; x += kAttnThreads)
      s_page[x] = (p0 + x < total_pages) ? trow[p0 + x] : -1;
  };

  // DMA of tile t into stage S: wave w moves key rows 8w .. 8w+7 of K and V.
  // Lane L of an instruction fills LDS chunk L % CHUNKS of row L / CHUNKS,
  // so it fetches logical chunk (L % CHUNKS) ^ swz(row); the element offset
  // of that chunk within a slot is fixed per lane and instruction.  Positions
  // outside the request read the zero block (the instruction is always
  // issued, which keeps the per-wave count of loads in flight fixed).
  // Positions are fetched in 16-byte chunks; pool offsets count chunks
  // (32-bit: the host checks that the pool holds fewer than 2^32 of them).
  const int row_chunks = Hkv * (D / 8);
  const unsigned pid_max = static_cast<unsigned>(num_slots >> pshift);   // last page id with a slot
  const unsigned nslots = static_cast<unsigned>(num_slots);
  int dma_row[C::IPW];
  int dma_col[C::IPW];
#pragma unroll
  for (int i = 0; i < C::IPW; ++i) {
    dma_row[i] = wave * 8 + i * C::KPI + l / C::CHUNKS;
    dma_col[i] = kvh * (D / 8) + ((l % C::CHUNKS) ^ swz<D>(dma_row[i]));
  }
  const uint4 *kp16 = reinterpret_cast<const uint4 *>(kpool);
  const uint4 *vp16 = reinterpret_cast<const uint4 *>(vpool);
  const uint32_t lds0 = lds_offset(smem);
  // LDS: a ring of four K tiles, then a ring of four V tiles.
  auto kbase = [&](int t) { return lds0 + (t & (kStages - 1)) * C::TILE_BYTES; };
  auto vbase = [&](int t) { return lds0 + (kStages + (t & (kStages - 1))) * C::TILE_BYTES; };
  // Pool addresses of this lane's chunks of tile t (K and V share them).
  auto tile_addr = [&](int t, const void *(&ka)[C::IPW], const void *(&va)[C::IPW]) {
    const int wbase = ((t / win_tiles) * win_tiles * kTile) >> pshift;
#pragma unroll
    for (int i = 0; i < C::IPW; ++i) {
      const int pos = t * kTile + dma_row[i];
      int idx = (pos >> pshift) - wbase;
      idx = idx < 0 ? 0 : (idx >= kPageCache ? kPageCache - 1 : idx);
      const int pid = s_page[idx];
      const unsigned slot = (static_cast<unsigned>(pid) << pshift) + static_cast<unsigned>(pos & pmask);
      const bool ok = (pos < total) & (static_cast<unsigned>(pid) <= pid_max) & (slot < nslots);
      const uint32_t off = slot * static_cast<uint32_t>(row_chunks) + dma_col[i];
      ka[i] = ok ? static_cast<const void *>(kp16 + off) : static_cast<const void *>(g_zero16);
      va[i] = ok ? static_cast<const void *>(vp16 + off) : static_cast<const void *>(g_zero16);
    }
  };
  auto issue = [&](uint32_t stage, const void *(&ga)[C::IPW]) {
#pragma unroll
    for (int i = 0; i < C::IPW; ++i)
      dma16(ga[i], __builtin_amdgcn_readfirstlane(stage + (wave * 8 + i * C::KPI) * C::ROW));
  };

  // Lane parts of the LDS fragment addresses (per stage: + stage base).
  // K: row 32*kh + 16*k2 + l16, chunk (4*ds + g4) ^ swz(row).
  // V^T (transposing read): row 32*kh + 16*k2 + 4*g4 + l16/4, 8 bytes at
  // d = 16*db + 4*(l16 % 4), i.e. chunk (2*db + (l16 % 4)/2) ^ swz(row).
  uint32_t koff[KB][C::DS], voff[KB][C::NO];
#pragma unroll
  for (int k2 = 0; k2 < KB; ++k2) {
    const int kr = 32 * kh + 16 * k2 + l16;
#pragma unroll
    for (int ds = 0; ds < C::DS; ++ds) koff[k2][ds] = kr * C::ROW + (((ds * 4 + g4) ^ swz<D>(kr)) << 4);
    const int vr = 32 * kh + 16 * k2 + 4 * g4 + (l16 >> 2);
#pragma unroll
    for (int db = 0; db < C::NO; ++db)
      voff[k2][db] = vr * C::ROW + (((2 * db + ((l16 & 3) >> 1)) ^ swz<D>(vr)) << 4) + ((l16 & 1) << 3);
  }

  // ---- S^T of tile t: A = K[key][d] (LDS), B = Q^T (registers)
  auto scores = [&](int t, f32x4 (&sc)[KB][RB]) {
    const uint32_t base = kbase(t);
#pragma unroll
    for (int k2 = 0; k2 < KB; ++k2)
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) sc[k2][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k2 = 0; k2 < KB; ++k2) {
#pragma unroll
      for (int ds = 0; ds < C::DS; ++ds) {
        const bf16x8 kf = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8 *>(base + koff[k2][ds]);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          sc[k2][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[rb][ds], sc[k2][rb], 0, 0, 0);
      }
    }
  };

  refresh_pages(0);
  __syncthreads();
  // the Q fragments and the page copy land here once, not inside the key loop
  __builtin_amdgcn_s_waitcnt(0);
  f32x4 s[KB][RB];
  // DMA schedule: K runs one tile ahead of V.  Step t issues K(t+4) and
  // V(t+3) (in that order); K(t+1) and V(t), which step t consumes, went out
  // together three steps earlier.  K(t+4) lands in the K slot that tile t's
  // scores (step t-1) last read, V(t+3) in the V slot of tile t-1's PV.
  const void *ka[C::IPW], *va[C::IPW], *va_next[C::IPW];
  if (ntiles > 0) {
    tile_addr(0, ka, va);
    issue(kbase(0), ka);
#pragma unroll
    for (int t0 = 1; t0 <= 3; ++t0) {
      tile_addr(t0, ka, va_next);
      issue(kbase(t0), ka);
      issue(vbase(t0 - 1), va);
#pragma unroll
      for (int i = 0; i < C::IPW; ++i) va[i] = va_next[i];
    }
    wait_vmcnt<6 * C::IPW>();            // K(0) is in
    __syncthreads();
    scores(0, s);
  }

  // Step t: softmax and PV of tile t, with the scores of tile t+1 computed
  // first so that their MFMAs run under the softmax's VALU work.
  // MASKED: tile t reaches past the prefix, so the tree mask applies.
  auto tile_step = [&](int t, auto MASKED) {
    constexpr bool masked = decltype(MASKED)::value;
    wait_vmcnt<4 * C::IPW>();            // this wave's K(t+1), V(t) are in (steps t-2, t-1 may fly)
    __syncthreads();                     // everyone's are; and the slots refilled below are no longer read
    if (t + 4 < ntiles && (t + 4) % win_tiles == 0) {   // block-uniform: next page window
      refresh_pages(t + 4);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
    tile_addr(t + 4, ka, va_next);
    issue(kbase(t + 4), ka);
    issue(vbase(t + 3), va);
#pragma unroll
    for (int i = 0; i < C::IPW; ++i) va[i] = va_next[i];
    const uint32_t base = vbase(t);

    // ---- mask, row max and the (rare) rescale of the running state
    // (lane: its row per rb; keys 16*k2 + 4*g4 + i)
    float v[RB][KB][4];
    float mneg[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
      for (int k2 = 0; k2 < KB; ++k2)
#pragma unroll
        for (int i = 0; i < 4; ++i) v[rb][k2][i] = s[k2][rb][i];
      if constexpr (masked) {
        const int kpos0 = t * kTile + 32 * kh + 4 * g4;
#pragma unroll
        for (int k2 = 0; k2 < KB; ++k2)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            // branch-free on purpose: a short-circuit form here becomes
            // divergent control flow whose -inf write lands in the MFMA
            // result register for every tree lane, visible ones included
            const int j = kpos0 + 16 * k2 + i - L;
            const uint32_t w = s_mask[nrel[rb]][(j >> 5) & 7];
            const bool vis =
                (j < 0) | ((static_cast<unsigned>(j) < static_cast<unsigned>(N)) & ((w >> (j & 31)) & 1u));
            v[rb][k2][i] = vis ? v[rb][k2][i] : -INFINITY;
          }
      }
      float rmax = fmaxf(fmaxf(fmaxf(v[rb][0][0], v[rb][0][1]), fmaxf(v[rb][0][2], v[rb][0][3])),
                         fmaxf(fmaxf(v[rb][1][0], v[rb][1][1]), fmaxf(v[rb][1][2], v[rb][1][3])));
      rmax = max_xor32(max_xor16(rmax));
      const float tmax = rmax * scale_log2;
      const bool need = tmax > m_run[rb] + 8.0f;
      if (__any(need)) {
        const float newm = need ? tmax : m_run[rb];
        const float alpha = need ? __builtin_amdgcn_exp2f(m_run[rb] - newm) : 1.0f;   // never -inf - -inf
        m_run[rb] = newm;
        l_run[rb] *= alpha;
#pragma unroll
        for (int j = 0; j < C::NO; ++j) {
          o[rb][j][0] *= alpha;
          o[rb][j][1] *= alpha;
          o[rb][j][2] *= alpha;
          o[rb][j][3] *= alpha;
        }
      }
      mneg[rb] = m_run[rb] == -INFINITY ? 0.f : -m_run[rb];
    }

    // ---- one straight-line block in a fixed order (in-order issue: an MFMA
    // runs while the VALU work after it issues).  The scores of tile t+1
    // (computed even past the last tile: the stage holds in-bounds data and
    // they go unused) are interleaved with the exponentials of tile t; then
    // O^T += V^T P^T with each pair of V reads issued one block ahead.
    const uint32_t nbase = kbase(t + 1);
    bf16x8 kf[KB][C::DS];
#pragma unroll
    for (int k2 = 0; k2 < KB; ++k2)
#pragma unroll
      for (int ds = 0; ds < C::DS; ++ds)
        kf[k2][ds] = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8 *>(nbase + koff[k2][ds]);
    f32x4 sn[KB][RB];
#pragma unroll
    for (int k2 = 0; k2 < KB; ++k2)
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) sn[k2][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
    __builtin_amdgcn_sched_barrier(0);
    float psum[RB] = {0.f, 0.f};
    bf16x8 pb[RB];
    constexpr int kSteps = KB * C::DS * RB / 2;          // two score MFMAs per step
    constexpr int kEps = RB * KB * 4 / kSteps;           // exponentials per step (2 or 4)
    static_assert(kEps * kSteps == RB * KB * 4 && kEps % 2 == 0, "even split of the exponentials");
#pragma unroll
    for (int st = 0; st < kSteps; ++st) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int m = 2 * st + h;                          // MFMA index: (k2, ds, rb)
        const int k2 = m / (C::DS * RB), ds = (m / RB) % C::DS, rb = m % RB;
        sn[k2][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[k2][ds], qf[rb][ds], sn[k2][rb], 0, 0, 0);
      }
      // exponentials of this lane's elements kEps*st .. +kEps-1 (rb, k2, i)
#pragma unroll
      for (int x = 0; x < kEps; x += 2) {
        const int e = kEps * st + x;
        const int rb = e / (KB * 4), k2 = (e / 4) % KB, i = e % 4;
        const float p0 = __builtin_amdgcn_exp2f(fmaf(v[rb][k2][i], scale_log2, mneg[rb]));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(v[rb][k2][i + 1], scale_log2, mneg[rb]));
        psum[rb] += p0 + p1;
        pb[rb][4 * k2 + i] = static_cast<__bf16>(p0);
        pb[rb][4 * k2 + i + 1] = static_cast<__bf16>(p1);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) l_run[rb] += psum[rb];

    // O^T += V^T P^T on MFMA 16x16x32.  MFMA k index 8*g4 + j stands for key
    // 4*g4 + j (j < 4) or 16 + 4*g4 + (j - 4) of this wave's 32 keys: P holds
    // them in that order, and the V^T operand is the two transposing reads
    // of the 16-key blocks side by side.  A transposing read: lane 4j + q of
    // a 16-lane group points at row j, d 4q..4q+3, and lane i of the group
    // receives d = i of the group's four rows.
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    auto vread = [&](int db) {
      const s16x4 a0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<lds_s16x4 *>(base + voff[0][db]));
      const s16x4 a1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<lds_s16x4 *>(base + voff[1][db]));
      bf16x8 a;
      __builtin_memcpy(reinterpret_cast<char *>(&a), &a0, 8);
      __builtin_memcpy(reinterpret_cast<char *>(&a) + 8, &a1, 8);
      return a;
    };
    bf16x8 va = vread(0);
#pragma unroll
    for (int db = 0; db < C::NO; ++db) {
      const bf16x8 vn = db + 1 < C::NO ? vread(db + 1) : va;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) o[rb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[rb], o[rb][db], 0, 0, 0);
      va = vn;
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int k2 = 0; k2 < KB; ++k2)
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) s[k2][rb] = sn[k2][rb];
  };

  // tiles wholly inside the prefix need no mask
  const int nfull = min(ntiles, L / kTile);
  int t = 0;
  for (; t < nfull; ++t) tile_step(t, std::false_type{});
  for (; t < ntiles; ++t) tile_step(t, std::true_type{});

  // ---- merge the two key halves of each row quarter (fixed order) and write
  __builtin_amdgcn_s_waitcnt(0);         // trailing DMAs (zero blocks) must land before reuse
  __syncthreads();
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    float lt = l_run[rb];
    lt = sum_xor32(sum_xor16(lt));
    if (g4 == 0) {
      s_m[kh][32 * rh + 16 * rb + l16] = m_run[rb];
      s_l[kh][32 * rh + 16 * rb + l16] = lt;
    }
  }
  __syncthreads();
  float fac[RB], mrow[RB], lrow[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int r = 32 * rh + 16 * rb + l16;
    const float M = fmaxf(s_m[0][r], s_m[1][r]);
    const float Mu = M == -INFINITY ? 0.f : M;
    const float Lsum = s_l[0][r] * exp2f(s_m[0][r] - Mu) + s_l[1][r] * exp2f(s_m[1][r] - Mu);
    fac[rb] = Lsum > 0.f ? exp2f(m_run[rb] - Mu) / Lsum : 0.f;
    mrow[rb] = Mu;
    lrow[rb] = Lsum;
  }
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int j = 0; j < C::NO; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) o[rb][j][i] *= fac[rb];

  // accumulator o[rb][db][i] holds row 32*rh+16*rb+l16 at d = 16*db + 4*g4 + i
  float *mbuf = reinterpret_cast<float *>(smem);
  if (kh == 1) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int db = 0; db < C::NO; ++db)
        *reinterpret_cast<float4 *>(mbuf + (32 * rh + 16 * rb + l16) * D + 16 * db + 4 * g4) =
            make_float4(o[rb][db][0], o[rb][db][1], o[rb][db][2], o[rb][db][3]);
  }
  __syncthreads();
  if (kh == 0) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int db = 0; db < C::NO; ++db) {
        float4 *p4 = reinterpret_cast<float4 *>(mbuf + (32 * rh + 16 * rb + l16) * D + 16 * db + 4 * g4);
        const float4 x = *p4;
        *p4 = make_float4(o[rb][db][0] + x.x, o[rb][db][1] + x.y, o[rb][db][2] + x.z, o[rb][db][3] + x.w);
      }
  }
  __syncthreads();
  for (int x = tid; x < kRows * (D / 8); x += kAttnThreads) {
    const int r = x / (D / 8), c8 = x % (D / 8);
    const int gr = row0 + r;
    const int node = gr / G, g = gr % G;
    if (node >= N) continue;
    const float4 a0 = *reinterpret_cast<const float4 *>(mbuf + r * D + c8 * 8);
    const float4 a1 = *reinterpret_cast<const float4 *>(mbuf + r * D + c8 * 8 + 4);
    const uint32_t w0 = f32_to_bf16_rne(a0.x) | (static_cast<uint32_t>(f32_to_bf16_rne(a0.y)) << 16);
    const uint32_t w1 = f32_to_bf16_rne(a0.z) | (static_cast<uint32_t>(f32_to_bf16_rne(a0.w)) << 16);
    const uint32_t w2 = f32_to_bf16_rne(a1.x) | (static_cast<uint32_t>(f32_to_bf16_rne(a1.y)) << 16);
    const uint32_t w3 = f32_to_bf16_rne(a1.z) | (static_cast<uint32_t>(f32_to_bf16_rne(a1.w)) << 16);
    *reinterpret_cast<uint4 *>(out + ((static_cast<int64_t>(b) * N + node) * Hq + kvh * G + g) * D + c8 * 8) =
        make_uint4(w0, w1, w2, w3);
  }
  if (lse && kh == 0 && g4 == 0) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int gr = row0 + 32 * rh + 16 * rb + l16;
      const int node = gr / G, g = gr % G;
      if (node < N)
        lse[(static_cast<int64_t>(b) * N + node) * Hq + kvh * G + g] =
            lrow[rb] > 0.f ? (mrow[rb] + log2f(lrow[rb])) * 0.69314718055994531f : -INFINITY;
    }
  }
}

template <int D>
int32_t launch_attn(int64_t blocks, hipStream_t st, const sdv_attn_shape &sh, int pshift, float scale_log2, int nrb,
                    const uint16_t *q, const uint16_t *k_pool, const uint16_t *v_pool,
                    const int32_t *page_table, const int32_t *prefix_len, const uint32_t *mask_bits, uint16_t *out,
                    float *lse) {
  const size_t lds = AttnCfg<D>::SMEM;
  static thread_local int configured_dev = -1;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(SDV_E_HIP, "tree_verify_attention: no device");
  if (configured_dev != dev) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(tree_attn_kernel<D>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return fail(SDV_E_HIP, "tree_verify_attention: LDS attribute: %s", hipGetErrorString(e));
    configured_dev = dev;
  }
  hipLaunchKernelGGL(tree_attn_kernel<D>, dim3(static_cast<unsigned>(blocks)), dim3(kAttnThreads), lds, st, sh.B,
                     sh.N, sh.Hq, sh.Hkv, pshift, sh.max_pages, sh.num_slots, scale_log2, nrb, q, k_pool,
                     v_pool, page_table, prefix_len, mask_bits, out, lse);
  return check_launch("tree_attn_kernel");
}

}  // namespace
}  // namespace sdv

using namespace sdv;

// Units of more than kRows query rows go to the wide kernel; its key split
// needs a workspace (sized for the split whether or not a call uses it).
static int wide_row_blocks(const sdv_attn_shape &sh) {
  const int rows = sh.N * (sh.Hq / sh.Hkv);
  return rows > kRows ? (rows + 255) / 256 : 0;
}

extern "C" size_t sdv_tree_verify_attention_workspace_size(sdv_attn_shape sh) {
  if (sh.B <= 0 || sh.N < 1 || sh.Hkv < 1 || sh.Hq % sh.Hkv != 0 || (sh.D != 64 && sh.D != 128)) return 0;
  const int nrb = wide_row_blocks(sh);
  return nrb ? attn_wide_workspace(static_cast<int64_t>(sh.B) * sh.Hkv * nrb, sh.D) : 0;
}

extern "C" int32_t sdv_tree_verify_attention(sdv_attn_shape sh, float sm_scale, const uint16_t *q,
                                             const uint16_t *k_pool, const uint16_t *v_pool,
                                             const int32_t *page_table, const int32_t *prefix_len,
                                             const uint32_t *mask_bits, uint16_t *out, float *lse, void *ws,
                                             size_t ws_bytes, void *stream) {
  clear_error();
  SDV_REQUIRE(sh.B >= 0 && sh.N >= 1 && sh.Hq >= 1 && sh.Hkv >= 1 && sh.page >= 1 && sh.max_pages >= 1 &&
                  sh.num_slots >= 0,
              SDV_E_SHAPE, "tree_verify_attention: bad sizes");
  SDV_REQUIRE(sh.Hq % sh.Hkv == 0, SDV_E_SHAPE, "tree_verify_attention: Hq %% Hkv != 0");
  SDV_REQUIRE(sh.D == 64 || sh.D == 128, SDV_E_UNSUPPORTED, "tree_verify_attention: D=%d not in {64,128}", sh.D);
  SDV_REQUIRE(sh.N <= 256 && sh.Hq / sh.Hkv <= 16, SDV_E_UNSUPPORTED,
              "tree_verify_attention: N <= 256 and Hq/Hkv <= 16 required");
  SDV_REQUIRE((sh.page & (sh.page - 1)) == 0 && sh.page <= (1 << 20), SDV_E_UNSUPPORTED,
              "tree_verify_attention: page=%d must be a power of two", sh.page);
  if (sh.B == 0) return SDV_OK;
  SDV_REQUIRE(q && k_pool && v_pool && page_table && prefix_len && mask_bits && out, SDV_E_NULL,
              "tree_verify_attention: NULL pointer");
  SDV_REQUIRE(reinterpret_cast<uintptr_t>(q) % 16 == 0 && reinterpret_cast<uintptr_t>(k_pool) % 16 == 0 &&
                  reinterpret_cast<uintptr_t>(v_pool) % 16 == 0 && reinterpret_cast<uintptr_t>(out) % 16 == 0,
              SDV_E_SHAPE, "tree_verify_attention: q, pools and out must be 16-byte aligned");
  SDV_REQUIRE(sh.num_slots >= 1, SDV_E_SHAPE, "tree_verify_attention: empty pool");
  int pshift = 0;
  while ((1 << pshift) < sh.page) ++pshift;
  SDV_REQUIRE(sh.num_slots + sh.page < (1LL << 31) && sh.num_slots * sh.Hkv * (sh.D / 8) < (1LL << 32),
              SDV_E_UNSUPPORTED, "tree_verify_attention: pool too large (2^31 slots, 2^32 16-byte chunks)");
  const float scale = sm_scale > 0.f ? sm_scale : 1.0f / sqrtf(static_cast<float>(sh.D));
  const float scale_log2 = scale * 1.4426950408889634f;
  hipStream_t st = as_stream(stream);
  const int wide_nrb = wide_row_blocks(sh);
  if (wide_nrb > 0) {
    // the persistent schedule when the caller gave its workspace
    const int64_t units = static_cast<int64_t>(sh.B) * sh.Hkv * wide_nrb;
    const size_t need = attn_wide_workspace(units, sh.D);
    const bool split = need > 0 && ws && ws_bytes >= need;
    SDV_REQUIRE(!split || reinterpret_cast<uintptr_t>(ws) % 256 == 0, SDV_E_WORKSPACE,
                "tree_verify_attention: workspace must be 256-byte aligned");
    return launch_attn_wide(st, sh, pshift, scale_log2, wide_nrb, split, q, k_pool, v_pool, page_table, prefix_len,
                            mask_bits, out, lse, ws);
  }
  const int G = sh.Hq / sh.Hkv;
  const int nrb = (sh.N * G + kRows - 1) / kRows;
  const int64_t units = static_cast<int64_t>(sh.B) * sh.Hkv;
  const int64_t units_pad = (units + kXcds - 1) / kXcds * kXcds;
  const int64_t blocks = units_pad * nrb;
  SDV_REQUIRE(blocks < (1LL << 31), SDV_E_UNSUPPORTED, "tree_verify_attention: grid too large");
  int32_t rc;
  if (sh.D == 64)
    rc = launch_attn<64>(blocks, st, sh, pshift, scale_log2, nrb, q, k_pool, v_pool, page_table, prefix_len,
                         mask_bits, out, lse);
  else
    rc = launch_attn<128>(blocks, st, sh, pshift, scale_log2, nrb, q, k_pool, v_pool, page_table, prefix_len,
                          mask_bits, out, lse);
  if (rc != SDV_OK) return rc;
  return check_launch("tree_attn_kernel");
}
