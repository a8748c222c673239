// A5 for units of more than 128 query rows: tree-verify attention -- one
// target pass over the prefix plus the candidate tree under the tree mask
// ("EAGLE speculative decoding in four parts", "Self-test" answer 1,
// "Exercises" question 1 and "Design trade-offs"; "[SGLang] Multi-Layer
// EAGLE" section 6, TARGET_VERIFY).  Same operation and arguments as the
// kernel in attn.hip, another work layout.
//
// Work layout.  A unit is one (request, KV head, block of 256 query rows)
// (row = node*G + g).  A workgroup of eight waves works on 256 rows of a
// unit, wave w rows 32w .. 32w+31 against all 64 keys of every tile, so
// each K/V tile is copied into LDS once for all of those rows (128-row
// workgroups would copy every tile twice).
//   * Schedule.  With a workspace, the grid is persistent (one workgroup per
//     CU at most): every unit weighs a fixed piece cost plus a cost per key
//     tile, the units of the length-ranked requests form one weighted
//     sequence, and workgroup ri takes the tiles whose start falls in the
//     ri-th of equal ranges of it (stream-K).  A unit cut between ranges
//     runs as several pieces; each piece keeps its partial softmax state
//     (m, l, O), and the piece that takes the unit's last ticket merges all
//     of them in range order, so the result does not depend on which piece
//     finished last.  The ranges of one XCD are consecutive, so a unit's
//     pieces share an L2.  Without a workspace, one workgroup per unit.
//   * K and V tiles move from the paged pool into LDS by DMA
//     (global_load_lds_dwordx4) through a ring of four K tiles and a ring of
//     four V tiles, the K stream one tile ahead; the chunk swizzle keeps the
//     MFMA fragment reads conflict free.
//   * Per step a wave issues the score MFMAs of tile t+1 and the PV MFMAs of
//     tile t, with the exponentials of tile t between them and the row
//     maxima of tile t+1 after the last PV MFMA.  The main loop is unrolled
//     over the four ring stages: every LDS fragment address is a fixed
//     per-lane register plus an immediate, and the scores alternate between
//     two register sets without copies.
//   * Each wave DMAs the page ids of the tile seven ahead into its own LDS
//     ring; a key's slot is clamped into the pool, and positions past the
//     request read its last token (finite data that the mask turns into a
//     zero weight), so every DMA reads real pool rows.
//   * The merge protocol: each piece takes a ticket (an atomic counter per
//     unit); the others publish their (m, l, O) in their workspace slots and
//     count themselves on a second counter after an agent-scope release; the
//     last waits for that count (bounded), merges, writes the output and
//     resets both counters to zero for the next call.  A wait that gives up
//     writes NaN rows and sets SDV_STATUS_ATTN_MERGE_WAIT in the workspace
//     header (the counters must then be reset by the host).
#include <type_traits>

#include "attn_common.hpp"

namespace sdv {
namespace {

constexpr int kWideRows = 256;            // query rows per workgroup (32 per wave)
constexpr unsigned kMergeSpin = 1u << 22; // polls before the merge gives up
// Persistent schedule weights: a key tile counts kTileWeight, the fixed cost
// of a piece (finding it, its prologue, the publish or merge of partial
// results) about seven tiles (measured on MI355X at B=32, Hq=32, Hkv=8,
// D=128: 2.1 us per tile, 2.5 us between pieces, 6.6 us prologue, 5 us
// publish or merge).
constexpr int kTileWeight = 4;
constexpr int kPieceWeight = 28;
constexpr int kMaxRanges = 512;           // workgroups of the persistent schedule at most
constexpr float kNoMax = -1e30f;          // running max before any visible key (finite: no inf - inf)

template <int D>
struct WideCfg : KvTile<D> {
  static constexpr int RB = 2;                             // 16-row blocks per wave
  static constexpr int KB = 4;                             // 16-key blocks per tile
  static constexpr int SMEM = KvTile<D>::RINGS;
  // partial O in bf16 (its relative rounding, 2^-9, is far inside the
  // output tolerance and halves the bytes a piece writes and the merge
  // reads), then (m, l) per row in fp32
  static constexpr size_t PART_O = static_cast<size_t>(kWideRows) * D * 2;
  static constexpr size_t PART = PART_O + kWideRows * 8;                      // + (m, l) per row
};

template <int N>
using IC = std::integral_constant<int, N>;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
constexpr bf16x2 kOnes2 = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};

// BIG: pools of 4 GiB or more (64-bit addresses per lane); otherwise a
// 32-bit byte offset per lane from the pool base in scalar registers.
template <int D, bool BIG>
__global__ void __launch_bounds__(kAttnThreads, 1)
tree_attn_wide_kernel(int B, int N, int Hq, int Hkv, int pshift, int max_pages, int64_t num_slots, float scale_log2,
                      int nrb, int nwg, const uint16_t *__restrict__ q,
                      const uint16_t *__restrict__ kpool, const uint16_t *__restrict__ vpool,
                      const int *__restrict__ table, const int *__restrict__ prefix_len,
                      const uint32_t *__restrict__ mask_bits, uint16_t *__restrict__ out, float *__restrict__ lse,
                      unsigned *__restrict__ sync, char *__restrict__ parts, unsigned *__restrict__ status,
                      unsigned wait_limit) {
  using C = WideCfg<D>;
  constexpr int RB = C::RB, KB = C::KB, DS = C::DS, NO = C::NO, IPW = C::IPW;
  constexpr int ROW = C::ROW, TILE = C::TILE_BYTES;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  __shared__ uint32_t s_mask[kWideRows][8];
  __shared__ int s_pid[8][kStages][kTile];   // per wave: page ids of four tiles (ring, by LDS DMA)
  __shared__ unsigned s_ticket;
  __shared__ int s_ok;
  __shared__ int s_req[kRankMax];           // request of each rank, longest prefix first
  __shared__ int s_len[kRankMax];           // prefix length of each request
  __shared__ int s_tpre[kRankMax + 1];      // weighted positions before each rank's units (persistent)
  __shared__ int s_rstart[kMaxRanges + 1];  // first weighted position of each range (persistent)
  __shared__ int s_wsum[kAttnThreads / kWave];
  __shared__ int s_meta[9];                 // the piece's values needed after its key loop

  const int G = Hq / Hkv;
  const int W = (N + 31) / 32;
  const int pmask = (1 << pshift) - 1;
  const int tid0 = threadIdx.x;
  const int upr = Hkv * nrb;                // units per request: KV head major, row block minor

  // ---- ranking: s_req[r] = the request of rank r (prefix length
  // descending, then index), for every rank at once
  const bool ranked = B <= kRankMax;
  if (ranked) {
    for (int i = tid0; i < B; i += kAttnThreads) s_len[i] = prefix_len[i];
    __syncthreads();
    for (int c = tid0; c < B; c += kAttnThreads) {
      const int Lc = s_len[c];
      int rk = 0;
      for (int o2 = 0; o2 < B; ++o2) {
        const int Lo = s_len[o2];
        rk += (Lo > Lc) | ((Lo == Lc) & (o2 < c));
      }
      s_req[rk] = c;
    }
    __syncthreads();
  }
  auto tiles_of_req = [&](int bq) __attribute__((always_inline)) {
    const int Lq = s_len[bq];
    const int64_t tq = static_cast<int64_t>(Lq) + N;
    const bool okq = Lq >= 0 && tq <= (static_cast<int64_t>(max_pages) << pshift);
    return okq ? static_cast<int>((tq + kTile - 1) / kTile) : 1;    // an unusable request: one empty piece
  };

  // ---- persistent schedule (nwg > 0).  Every unit of nt key tiles weighs
  // kPieceWeight + kTileWeight * nt (the fixed cost of a piece, then its
  // tiles): its tile k starts at weighted position C_u + kPieceWeight +
  // kTileWeight * k.  The units, rank by rank, form one sequence of Tw
  // positions, cut into nwg equal ranges; a range takes the tiles whose start
  // lies in it.  Range ri goes to hardware block (ri % (nwg/8)) * 8 +
  // ri / (nwg/8), so the ranges of one XCD are consecutive and the pieces of
  // a unit share its L2.
  int Tw = 0;
  if (nwg > 0) {
    // exclusive scan of the ranks' weights, two ranks per thread
    const int r0 = 2 * tid0;
    const int l0 = tid0 & (kWave - 1), w0 = tid0 / kWave;
    const int t0 = r0 < B ? upr * (kPieceWeight + kTileWeight * tiles_of_req(s_req[r0])) : 0;
    const int t1 = r0 + 1 < B ? upr * (kPieceWeight + kTileWeight * tiles_of_req(s_req[r0 + 1])) : 0;
    int inc = t0 + t1;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int y = __shfl_up(inc, off, kWave);
      if (l0 >= off) inc += y;
    }
    if (l0 == kWave - 1) s_wsum[w0] = inc;
    __syncthreads();
    int before = 0;
    for (int w2 = 0; w2 < w0; ++w2) before += s_wsum[w2];
    const int excl = before + inc - (t0 + t1);
    if (r0 <= B) s_tpre[r0] = excl;
    if (r0 + 1 <= B) s_tpre[r0 + 1] = excl + t0;
    __syncthreads();
    Tw = __builtin_amdgcn_readfirstlane(s_tpre[B]);
    for (int r = tid0; r <= nwg; r += kAttnThreads)
      s_rstart[r] = static_cast<int>(static_cast<int64_t>(r) * Tw / nwg);
    __syncthreads();
  }
  const int per_xcd = nwg / kXcds;
  const int ri = nwg > 0 ? (static_cast<int>(blockIdx.x) % kXcds) * per_xcd + static_cast<int>(blockIdx.x) / kXcds : 0;
  auto range_start = [&](int r) __attribute__((always_inline)) { return __builtin_amdgcn_readfirstlane(s_rstart[r]); };
  // the range holding weighted position x (the last of equal starts)
  auto range_of = [&](int x) __attribute__((always_inline)) {
    int lo = 0, hi = nwg;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (range_start(mid) <= x) lo = mid; else hi = mid;
    }
    return lo;
  };
  // tiles of a unit (first tile starting at S0) whose start lies before x
  auto tiles_before = [&](int x, int S0, int nt) __attribute__((always_inline)) {
    return x <= S0 ? 0 : min(nt, (x - S0 + kTileWeight - 1) / kTileWeight);
  };
  const int my_lo = nwg > 0 ? range_start(ri) : 0;
  const int my_hi = nwg > 0 ? range_start(ri + 1) : 1;

  // ---- pieces: [tb, te) of one unit's tiles.  Without the persistent
  // schedule, block h owns one whole unit: the units of one XCD are its
  // rank-ordered ones, the row blocks of a unit consecutive.
  int cur = my_lo;
  auto piece = [&]() __attribute__((always_inline)) {
    int b, kvh, rblk, tb, te_raw, uidx, npieces = 1, slot_first = 0, slot_last = 0, S0 = 0;
    if (nwg > 0) {
      int lo = 0, hi = B;                        // the rank r with s_tpre[r] <= cur < s_tpre[r+1]
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (__builtin_amdgcn_readfirstlane(s_tpre[mid]) <= cur) lo = mid; else hi = mid;
      }
      const int r = lo;
      const int pre_r = __builtin_amdgcn_readfirstlane(s_tpre[r]);
      const int wu = (__builtin_amdgcn_readfirstlane(s_tpre[r + 1]) - pre_r) / upr;   // weight of one unit
      const int nt = (wu - kPieceWeight) / kTileWeight;
      const int uir = (cur - pre_r) / wu;
      const int C_u = pre_r + uir * wu;
      S0 = C_u + kPieceWeight;
      tb = tiles_before(cur, S0, nt);
      te_raw = tiles_before(my_hi, S0, nt);
      b = __builtin_amdgcn_readfirstlane(s_req[r]);
      kvh = uir / nrb;
      rblk = uir % nrb;
      uidx = r * upr + uir;
      // the unit's pieces: the ranges holding the start of one of its tiles
      slot_first = range_of(S0);
      slot_last = range_of(S0 + kTileWeight * (nt - 1));
      npieces = 0;
      for (int rr = slot_first; rr <= slot_last; ++rr)
        npieces += tiles_before(range_start(rr + 1), S0, nt) > tiles_before(range_start(rr), S0, nt) ? 1 : 0;
      cur = min(my_hi, C_u + wu);
    } else {
      const int xcd = blockIdx.x % kXcds;
      const int slot_in_xcd = blockIdx.x / kXcds;
      const int rank = (slot_in_xcd / nrb) * kXcds + xcd;
      rblk = slot_in_xcd % nrb;
      cur = my_hi;
      if (rank >= B * Hkv) return;
      b = ranked ? __builtin_amdgcn_readfirstlane(s_req[rank / Hkv]) : rank / Hkv;
      kvh = rank % Hkv;
      tb = 0;
      te_raw = 1 << 30;
      uidx = rank * nrb + rblk;
    }
    if (tb >= te_raw) return;                // no tile of the unit starts in this range
    b = __builtin_amdgcn_readfirstlane(b);
    kvh = __builtin_amdgcn_readfirstlane(kvh);
    rblk = __builtin_amdgcn_readfirstlane(rblk);
    tb = __builtin_amdgcn_readfirstlane(tb);
    te_raw = __builtin_amdgcn_readfirstlane(te_raw);
    npieces = __builtin_amdgcn_readfirstlane(npieces);
    slot_first = __builtin_amdgcn_readfirstlane(slot_first);
    slot_last = __builtin_amdgcn_readfirstlane(slot_last);
    uidx = __builtin_amdgcn_readfirstlane(uidx);
    const int tid = threadIdx.x;
    const int wave = tid / kWave;
    const int l = lane_id();
    const int l16 = l & 15;
    const int g4 = l >> 4;

  const int L = ranked ? s_len[b] : prefix_len[b];
  const int total = L + N;
  const int *trow = table + static_cast<int64_t>(b) * max_pages;
  const bool req_ok = L >= 0 && static_cast<int64_t>(total) <= (static_cast<int64_t>(max_pages) << pshift);
  const int ntiles = req_ok ? (total + kTile - 1) / kTile : 0;
  const int te = min(te_raw, ntiles);
  const int nfull = min(te, L / kTile);     // tiles below nfull lie wholly inside the prefix

  const int row0 = rblk * kWideRows;
  const int node0 = row0 / G;
  for (int x = tid; x < kWideRows * 8; x += kAttnThreads) {
    const int nn = x / 8, w = x % 8;
    uint32_t v = 0;
    if (node0 + nn < N && w < W) v = mask_bits[(static_cast<int64_t>(b) * N + node0 + nn) * W + w];
    s_mask[nn][w] = v;
  }

  // this lane's rows: row0 + 32*wave + 16*rb + l16
  int nrel[RB];
  bf16x8 qf[RB][DS];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int r = row0 + 32 * wave + 16 * rb + l16;
    const int node = r / G, g = r % G;
    nrel[rb] = node - node0;
    const bool ok = node < N;
    const uint16_t *qp = q + ((static_cast<int64_t>(b) * N + (ok ? node : 0)) * Hq + kvh * G + g) * D;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      uint4 u = ok ? *reinterpret_cast<const uint4 *>(qp + ds * 32 + 8 * g4) : make_uint4(0, 0, 0, 0);
      __builtin_memcpy(&qf[rb][ds], &u, 16);
    }
  }
  f32x4 o[RB][NO];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int j = 0; j < NO; ++j) o[rb][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[RB], l_run[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m_run[rb] = kNoMax;
    l_run[rb] = 0.f;
  }

  // ---- DMA.  Wave w moves key rows 8w .. 8w+7 of a tile: lane L of an
  // instruction fills LDS chunk L % CHUNKS of row L / CHUNKS, so it fetches
  // logical chunk (L % CHUNKS) ^ swz(row).  A key's address is the pool base
  // plus slot * (bytes per slot) plus this lane's chunk.
  const uint32_t slot_bytes = static_cast<uint32_t>(Hkv) * D * 2;
  const unsigned nslots = static_cast<unsigned>(num_slots);
  const unsigned pid_max = static_cast<unsigned>((num_slots - 1) >> pshift);   // last page id with a slot
  int dma_row[IPW];
  uint32_t col_bytes[IPW];
#pragma unroll
  for (int i = 0; i < IPW; ++i) {
    dma_row[i] = wave * 8 + i * C::KPI + l / C::CHUNKS;
    col_bytes[i] = 16u * (kvh * (D / 8) + ((l % C::CHUNKS) ^ swz<D>(dma_row[i])));
  }
  const uint32_t lds0 = lds_offset(smem);
  const uint32_t m0k = __builtin_amdgcn_readfirstlane(lds0 + wave * 8 * ROW);   // this wave's rows, K ring
  const uint32_t m0v = m0k + kStages * TILE;                                     // V ring
  const uint32_t m0p = __builtin_amdgcn_readfirstlane(lds_offset(&s_pid[wave][0][0]));   // page-id ring

  // Key position that row r of tile t reads: its own, clamped to the
  // request's last token; tiles past this chunk (the pipeline runs three
  // ahead) all read that last token, one row that stays in L2.
  auto key_pos = [&](int t, int r) __attribute__((always_inline)) { return t < te ? min(t * kTile + r, total - 1) : total - 1; };
  // Page ids of every position of tile t into ring slot u of this wave (one
  // instruction: lane L takes key_pos(t, L)).
  auto pid_dma = [&](int t, int u) __attribute__((always_inline)) {
    const int idx = key_pos(t, l) >> pshift;
    dma4(trow + idx, m0p + u * kTile * 4);
  };
  // Page ids of this lane's rows of tile t (ring slot u), then their pool slots.
  auto read_pids = [&](int u, int (&pid)[IPW]) {
#pragma unroll
    for (int i = 0; i < IPW; ++i) pid[i] = s_pid[wave][u][dma_row[i]];
  };
  auto tile_off = [&](int t, const int (&pids)[IPW], uint32_t (&slot)[IPW]) {
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const int pos = key_pos(t, dma_row[i]);
      const unsigned pid = min(static_cast<unsigned>(pids[i]), pid_max);
      slot[i] = min((pid << pshift) + static_cast<unsigned>(pos & pmask), nslots - 1);
    }
  };
  auto issue = [&](uint32_t m0, const uint16_t *pool, const uint32_t (&slot)[IPW]) {
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      if constexpr (BIG) {
        const uint64_t a = reinterpret_cast<uint64_t>(pool) + static_cast<uint64_t>(slot[i]) * slot_bytes + col_bytes[i];
        dma16(reinterpret_cast<const void *>(a), m0 + i * C::KPI * ROW);
      } else {
        dma16s(slot[i] * slot_bytes + col_bytes[i], pool, m0 + i * C::KPI * ROW);
      }
    }
  };

  // ---- LDS fragment addresses: a per-lane register plus an immediate
  // (ring stage * TILE + key block * 16 rows).
  // K (A operand of S^T = K Q^T): key row 16*kb + l16, chunk (4*ds + g4) ^ swz(row).
  // V^T (transposing read): key row 16*kb + 4*g4 + l16/4, 8 bytes at
  // d = 16*db + 4*(l16 % 4), i.e. chunk (2*db + (l16 % 4)/2) ^ swz(row).
  uint32_t koff[DS], voff[NO];
#pragma unroll
  for (int ds = 0; ds < DS; ++ds) koff[ds] = lds0 + l16 * ROW + (((ds * 4 + g4) ^ swz<D>(l16)) << 4);
  {
    const int vr = 4 * g4 + (l16 >> 2);
#pragma unroll
    for (int db = 0; db < NO; ++db)
      voff[db] = lds0 + kStages * TILE + vr * ROW + (((2 * db + ((l16 & 3) >> 1)) ^ swz<D>(vr)) << 4) +
                 ((l16 & 1) << 3);
  }
  typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  auto kread = [&](uint32_t kst, int kb, int ds) __attribute__((always_inline)) {
    return *reinterpret_cast<const lds_bf16x8 *>(koff[ds] + kst + kb * 16 * ROW);
  };
  // V^T operand of 32 keys (key blocks 2kk, 2kk+1) and d block db.  A
  // transposing read: lane 4j + q of a 16-lane group points at row j, d
  // 4q..4q+3, and lane i of the group receives d = i of the group's four rows.
  auto vread = [&](uint32_t vst, int kk, int db) __attribute__((always_inline)) {
    const s16x4 a0 =
        __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<lds_s16x4 *>(voff[db] + vst + 2 * kk * 16 * ROW));
    const s16x4 a1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        reinterpret_cast<lds_s16x4 *>(voff[db] + vst + (2 * kk + 1) * 16 * ROW));
    bf16x8 a;
    __builtin_memcpy(reinterpret_cast<char *>(&a), &a0, 8);
    __builtin_memcpy(reinterpret_cast<char *>(&a) + 8, &a1, 8);
    return a;
  };

  // ---- softmax state.  sc holds one tile's S^T blocks sc[kb][rb] (lane
  // (g4, l16): keys 16*kb + 4*g4 + i of row block rb's row l16); a step
  // overwrites them with the next tile's, key block by key block, once the
  // exponentials that read them have run.
  static_assert(KB == 4, "the step order below covers four key blocks");
  f32x4 sc[KB][RB];
  bf16x8 pb[RB][2];                      // P of the current tile, bf16, one per 32-key PV block

  // mask of key blocks kb, kb+1 of tile t (tiles reaching into the tree)
  auto mask_pair = [&](int t, int kb0) __attribute__((always_inline)) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int kpos0 = t * kTile + 4 * g4 - L;
#pragma unroll
      for (int kb = kb0; kb < kb0 + 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          // branch-free on purpose: a short-circuit form becomes divergent
          // control flow whose -inf write can land in the MFMA result
          // register for every lane
          const int j = kpos0 + 16 * kb + i;
          const uint32_t w = s_mask[nrel[rb]][(j >> 5) & 7];
          const bool vis =
              (j < 0) | ((static_cast<unsigned>(j) < static_cast<unsigned>(N)) & ((w >> (j & 31)) & 1u));
          sc[kb][rb][i] = vis ? sc[kb][rb][i] : -INFINITY;
        }
    }
  };
  // maximum of this lane's 8 values in key blocks kb, kb+1 (3-input
  // maximum trees, no NaN quieting in between)
  auto pair_max = [&](int kb0, float (&pm)[RB]) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const f32x4 &a = sc[kb0][rb], &c = sc[kb0 + 1][rb];
      pm[rb] = vmax(vmax(vmax(vmax(a[0], a[1]), a[2]), vmax(vmax(a[3], c[0]), c[1])), vmax(c[2], c[3]));
    }
  };
  // Row maxima across the four lane groups, in log2 units.
  auto row_max = [&](const float (&p0)[RB], const float (&p1)[RB], float (&tmax)[RB]) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) tmax[rb] = max_xor32(max_xor16(vmax(p0[rb], p1[rb]))) * scale_log2;
  };
  // The running state moves to a new reference max only when a score
  // exceeds the current one by more than 2^8 (rare): m, l and the exponent
  // here, branch-free; O by rescale_o once its MFMAs are done.
  auto update_state = [&](const float (&tmax)[RB], float (&alpha)[RB]) {
    bool anyneed = false;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const bool need = tmax[rb] > m_run[rb] + 8.0f;
      const float newm = need ? tmax[rb] : m_run[rb];
      alpha[rb] = need ? __builtin_amdgcn_exp2f(m_run[rb] - newm) : 1.0f;   // both finite
      m_run[rb] = newm;
      l_run[rb] *= alpha[rb];
      anyneed |= need;
    }
    return anyneed;
  };
  auto rescale_o = [&](bool anyneed, const float (&alpha)[RB]) {
    if (__any(anyneed)) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int j = 0; j < NO; ++j) {
          o[rb][j][0] *= alpha[rb];
          o[rb][j][1] *= alpha[rb];
          o[rb][j][2] *= alpha[rb];
          o[rb][j][3] *= alpha[rb];
        }
    }
  };

  // Exponentials of this lane's element pair x (0..15) of key block kb:
  // (rb = x / 2, i = 2 * (x % 2)) -> P in bf16 for PV block kb / 2; the row
  // sum adds the pair as rounded to bf16 (one dot2 with (1, 1)), the weights
  // the PV product uses.
  auto exp_pair = [&](int kb, int x) __attribute__((always_inline)) {
    const int rb = x / 2, i = 2 * (x % 2), kk = kb / 2, e = 4 * (kb % 2) + i;
    const float q0 = __builtin_amdgcn_exp2f(fmaf(sc[kb][rb][i], scale_log2, -m_run[rb]));
    const float q1 = __builtin_amdgcn_exp2f(fmaf(sc[kb][rb][i + 1], scale_log2, -m_run[rb]));
    bf16x2 pk;
    pk[0] = static_cast<__bf16>(q0);
    pk[1] = static_cast<__bf16>(q1);
    l_run[rb] = __builtin_amdgcn_fdot2_f32_bf16(pk, kOnes2, l_run[rb], false);
    pb[rb][kk][e] = pk[0];
    pb[rb][kk][e + 1] = pk[1];
  };
  // exponential pairs [x0, x1) of the 16 (kb, x) pairs of key blocks kb0 ..
  auto exps = [&](int kb0, int x0, int x1) __attribute__((always_inline)) {
#pragma unroll
    for (int x = x0; x < x1; ++x) exp_pair(kb0 + x / 4, x % 4);
  };
  // items 0 .. n-1 spread evenly over `iters` iterations: those of iteration it
  auto spread = [](int n, int iters, int it, auto &&fn) __attribute__((always_inline)) {
#pragma unroll
    for (int x = it * n / iters; x < (it + 1) * n / iters; ++x) fn(x);
  };

  // ---- scores of key block kb of a tile from K stage kst into sc[kb]
  // (fragment ds of the block in kf when called; the next block's first
  // fragment is read into kf on the way out when `more`), VALU work
  // valu(ds) after each pair of MFMAs
  auto score_block = [&](uint32_t kst, int kb, bf16x8 &kf, bool more, auto &&valu) __attribute__((always_inline)) {
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      const bf16x8 cur = kf;
      if (ds + 1 < DS)
        kf = kread(kst, kb, ds + 1);
      else if (more)
        kf = kread(kst, kb + 1, 0);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
        sc[kb][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cur, qf[rb][ds],
                                                             ds == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : sc[kb][rb], 0, 0,
                                                             0);
      valu(ds);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // O^T += V^T P^T for PV block kk from V stage vst (its first operand in va
  // when called), VALU work valu(db) after each pair of MFMAs
  auto pv_block = [&](uint32_t vst, int kk, bf16x8 &va, auto &&valu) __attribute__((always_inline)) {
#pragma unroll
    for (int db = 0; db < NO; ++db) {
      const bf16x8 cur = va;
      if (db + 1 < NO) va = vread(vst, kk, db + 1);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
        o[rb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cur, pb[rb][kk], o[rb][db], 0, 0, 0);
      valu(db);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ---- one step: softmax and PV of tile t (masked scores in sc, its row
  // maxima applied), scores and row maxima of tile t+1.  STAGE: ring slot of
  // tile t.
  uint32_t offv[IPW];      // V chunk offsets of the tile whose K went out last step
  // DMA batches: step t issues K(t+4) and V(t+3) (LDS slots of K(t) and
  // V(t-1), read in step t-1) and the page ids of tile t+7 (ring slot of
  // tile t+3's, read in step t-1); it needs K(t+1), V(t) and the page ids of
  // tile t+4, which went out together three steps earlier.
  constexpr int kBatch = 1 + 2 * IPW;    // vector-memory instructions per step and wave
  auto step = [&](int t, auto STAGE) __attribute__((always_inline)) {
    constexpr int S = decltype(STAGE)::value;
    wait_vmcnt<2 * kBatch>();            // this wave's batch of step t-3 is in (two later ones may fly)
    __syncthreads();                     // everyone's are; and the slots refilled below are no longer read
    // This step's DMA batch goes out in pieces between MFMAs (a stalled
    // issue then overlaps matrix work): K(t+4) after the first score MFMAs,
    // V(t+3) after the next ones, the page ids of tile t+7 during PV block 0.
    int pids[IPW];
    read_pids(S, pids);                  // page ids of tile t+4, in by the wait above
    uint32_t offn[IPW];
    auto issue_k = [&]() __attribute__((always_inline)) {
      tile_off(t + 4, pids, offn);
      issue(m0k + S * TILE, kpool, offn);                                            // K(t+4)
    };
    auto issue_v = [&]() __attribute__((always_inline)) {
      issue(m0v + ((S + kStages - 1) & (kStages - 1)) * TILE, vpool, offv);          // V(t+3)
#pragma unroll
      for (int i = 0; i < IPW; ++i) offv[i] = offn[i];
    };
    constexpr uint32_t kst = ((S + 1) & (kStages - 1)) * TILE;    // K(t+1)
    constexpr uint32_t vst = S * TILE;                             // V(t)
    const bool next = t + 1 < te;                                  // block-uniform
    const bool masked_next = t + 1 >= nfull;
    bf16x8 kf = kread(kst, 0, 0);
    auto none = [](int) __attribute__((always_inline)) {};
    // (key block 0's exponentials ran at the end of the last step)
    // 1.-2. scores of key blocks 0, 1 of tile t+1 | exponentials of key blocks 1, 2 (first half)
    score_block(kst, 0, kf, true, [&](int ds) __attribute__((always_inline)) {
      spread(4, DS, ds, [&](int x) __attribute__((always_inline)) { exp_pair(1, x); });
      if (ds == 0) issue_k();
    });
    bf16x8 va = vread(vst, 0, 0);
    score_block(kst, 1, kf, false, [&](int ds) __attribute__((always_inline)) {
      spread(2, DS, ds, [&](int x) __attribute__((always_inline)) { exp_pair(2, x); });
      if (ds == 0) issue_v();
    });
    // 3. PV block 0 | exponentials of key block 2 (second half), 3 (first half)
    kf = kread(kst, 2, 0);
    pv_block(vst, 0, va, [&](int db) __attribute__((always_inline)) {
      spread(4, NO, db, [&](int x) __attribute__((always_inline)) { exp_pair(x < 2 ? 2 : 3, (x + 2) % 4); });   // block 2 pairs 2, 3; block 3 pairs 0, 1
      if (db == 0) pid_dma(t + 7, (S + 3) & (kStages - 1));
    });
    va = vread(vst, 1, 0);
    // 4.-5. scores of key blocks 2, 3 | exponentials of key block 3 (second
    // half); mask and maxima of key blocks 0, 1 of tile t+1
    float p0[RB], p1[RB], tmax[RB], alpha[RB];
    score_block(kst, 2, kf, true, [&](int ds) __attribute__((always_inline)) { spread(2, DS, ds, [&](int x) __attribute__((always_inline)) { exp_pair(3, 2 + x); }); });
    score_block(kst, 3, kf, false, [&](int ds) __attribute__((always_inline)) {
      if (ds == 0 && masked_next) mask_pair(t + 1, 0);
      if (ds == DS - 1) pair_max(0, p0);
    });
    // 6. PV block 1 | tile t+1: mask and maxima of key blocks 2, 3, row
    // maxima, the state update, exponentials of key block 0; then the (rare)
    // rescale of O
    if (next) {
      bool anyneed = false;
      pv_block(vst, 1, va, [&](int db) __attribute__((always_inline)) {
        spread(8, NO, db, [&](int x) __attribute__((always_inline)) {
          switch (x) {
            case 0: if (masked_next) mask_pair(t + 1, 2); break;
            case 1: pair_max(2, p1); break;
            case 2: row_max(p0, p1, tmax); break;
            case 3: anyneed = update_state(tmax, alpha); break;
            case 4: exps(0, 0, 1); break;
            case 5: exps(0, 1, 2); break;
            case 6: exps(0, 2, 3); break;
            default: exps(0, 3, 4); break;
          }
        });
      });
      rescale_o(anyneed, alpha);
    } else {
      pv_block(vst, 1, va, none);
    }
  };

  // ---- prologue: page ids of tiles tb .. tb+3 (in flight with the Q
  // fragments and the mask), K(tb), then three batches shaped like a step's:
  // page ids of tile tb+4+u, K(tb+1+u), V(tb+u)
  if (tb < te) {
#pragma unroll
    for (int u = 0; u < kStages; ++u) pid_dma(tb + u, u);
  }
  __syncthreads();
  __builtin_amdgcn_s_waitcnt(0);         // Q, the mask and the page ids land here, not in the key loop
  if (tb < te) {
    uint32_t off[kStages][IPW];
#pragma unroll
    for (int u = 0; u < kStages; ++u) {
      int pids[IPW];
      read_pids(u, pids);
      tile_off(tb + u, pids, off[u]);
    }
    __builtin_amdgcn_s_waitcnt(0);       // page ids read before their slots are refilled
    issue(m0k, kpool, off[0]);
#pragma unroll
    for (int u = 0; u + 1 < kStages; ++u) {
      issue(m0k + (u + 1) * TILE, kpool, off[u + 1]);
      issue(m0v + u * TILE, vpool, off[u]);
      pid_dma(tb + 4 + u, u);
    }
#pragma unroll
    for (int i = 0; i < IPW; ++i) offv[i] = off[kStages - 1][i];
    wait_vmcnt<3 * kBatch>();            // K(tb) is in
    __syncthreads();
    bf16x8 kf = kread(0, 0, 0);
    auto none = [](int) __attribute__((always_inline)) {};
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) score_block(0, kb, kf, kb + 1 < KB, none);
    float p0[RB], p1[RB], tmax[RB], alpha[RB];
    if (tb >= nfull) {
      mask_pair(tb, 0);
      mask_pair(tb, 2);
    }
    pair_max(0, p0);
    pair_max(2, p1);
    row_max(p0, p1, tmax);
    update_state(tmax, alpha);           // O is still zero: nothing to rescale
    exps(0, 0, 4);
  }

  // The values the merge and the output need wait in LDS during the key
  // loop, which needs every register it can get.
  if (tid == 0) {
    s_meta[0] = npieces;
    s_meta[1] = slot_first;
    s_meta[2] = slot_last;
    s_meta[3] = S0;
    s_meta[4] = uidx;
    s_meta[5] = b;
    s_meta[6] = kvh;
    s_meta[7] = row0;
    s_meta[8] = ntiles;
  }
  // ---- main loop: the step of tile t uses ring stage (t - tb) % 4; the
  // loop leaves after any step
  for (int t = tb; t < te;) {
    step(t, IC<0>{});
    if (++t >= te) break;
    step(t, IC<1>{});
    if (++t >= te) break;
    step(t, IC<2>{});
    if (++t >= te) break;
    step(t, IC<3>{});
    ++t;
  }
  __builtin_amdgcn_s_waitcnt(0);         // trailing DMAs land before the workgroup ends
  __syncthreads();
  const int m_np = __builtin_amdgcn_readfirstlane(s_meta[0]);
  const int m_sf = __builtin_amdgcn_readfirstlane(s_meta[1]);
  const int m_sl = __builtin_amdgcn_readfirstlane(s_meta[2]);
  const int m_S0 = __builtin_amdgcn_readfirstlane(s_meta[3]);
  const int m_uidx = __builtin_amdgcn_readfirstlane(s_meta[4]);
  const int m_b = __builtin_amdgcn_readfirstlane(s_meta[5]);
  const int m_kvh = __builtin_amdgcn_readfirstlane(s_meta[6]);
  const int m_row0 = __builtin_amdgcn_readfirstlane(s_meta[7]);
  const int m_nt = __builtin_amdgcn_readfirstlane(s_meta[8]);

  // ---- row sums over the four lane groups (m_run is equal across them)
  float lrow[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) lrow[rb] = sum_xor32(sum_xor16(l_run[rb]));
  float mfin[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) mfin[rb] = m_run[rb];

  bool emit = true;
  if (m_np > 1) {
    // The unit's pieces run on the non-empty ranges m_sf ..
    // m_sl.  The piece of range rr keeps its partial in slot 2*rr + 1
    // when rr starts before the unit (the unit is rr's last piece), else in
    // slot 2*rr.  The piece that takes the last ticket merges every piece in
    // range order, so the result does not depend on which one finished last;
    // the others publish and count themselves on `done`.
    unsigned *ticket = sync + 2 * static_cast<int64_t>(m_uidx);
    unsigned *done = ticket + 1;
    const int nt_u = m_nt > 0 ? m_nt : 1;
    // range rr holds a piece of the unit iff a tile of it starts there; the
    // piece is rr's first one (slot 2*rr) when the unit's first tile starts
    // before rr, else it is rr's last one (slot 2*rr + 1)
    auto slot_ptr = [&](int rr) __attribute__((always_inline)) {
      const int sl = 2 * rr + (m_S0 < range_start(rr) ? 0 : 1);
      return parts + static_cast<int64_t>(sl) * C::PART;
    };
    auto nonempty = [&](int rr) __attribute__((always_inline)) {
      return tiles_before(range_start(rr + 1), m_S0, nt_u) > tiles_before(range_start(rr), m_S0, nt_u);
    };
    if (tid == 0) s_ticket = __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (s_ticket + 1 < static_cast<unsigned>(m_np)) {
      uint2 *pO = reinterpret_cast<uint2 *>(slot_ptr(ri));
      float2 *pml = reinterpret_cast<float2 *>(slot_ptr(ri) + C::PART_O);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int db = 0; db < NO; ++db)
          pO[((wave * RB + rb) * NO + db) * kWave + l] =
              make_uint2(f32_to_bf16_rne(o[rb][db][0]) | (static_cast<uint32_t>(f32_to_bf16_rne(o[rb][db][1])) << 16),
                         f32_to_bf16_rne(o[rb][db][2]) | (static_cast<uint32_t>(f32_to_bf16_rne(o[rb][db][3])) << 16));
      if (g4 == 0) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) pml[wave * 32 + 16 * rb + l16] = make_float2(mfin[rb], lrow[rb]);
      }
      // every wave's stores complete (stores count in vmcnt), then one
      // agent-scope release (one L2 write-back for the workgroup) before the
      // count moves
      wait_vmcnt<0>();
      __syncthreads();
      if (tid == 0) __hip_atomic_fetch_add(done, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
      emit = false;
    } else {
      // last: wait for the others' partials, then reset both counters for the next call
      if (tid == 0) {
        int ok = 0;
        for (unsigned spins = 0; spins < wait_limit; ++spins) {
          if (__hip_atomic_load(done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1 >=
              static_cast<unsigned>(m_np)) {
            ok = 1;
            break;
          }
          __builtin_amdgcn_s_sleep(2);
        }
        if (!ok) raise_status(status, SDV_STATUS_ATTN_MERGE_WAIT);
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        __hip_atomic_store(ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_ok = ok;
      }
      __syncthreads();                   // thread 0's acquire covers the workgroup (one CU, one L1)
      // merge in piece order: m = max, l and O summed with weights 2^(m_p - m)
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        float Mu = mfin[rb];
        for (int pp = m_sf; pp <= m_sl; ++pp) {
          if (pp == ri || !nonempty(pp)) continue;
          const float2 *pml = reinterpret_cast<const float2 *>(slot_ptr(pp) + C::PART_O);
          Mu = fmaxf(Mu, pml[wave * 32 + 16 * rb + l16].x);    // finite: maxima start at kNoMax
        }
        f32x4 acc[NO];
        float lacc = 0.f;
        bool first = true;
        for (int pp = m_sf; pp <= m_sl; ++pp) {
          if (!nonempty(pp)) continue;
          float mp, lp;
          f32x4 xo[NO];
          if (pp == ri) {
            // its own partial as the others see it (rounded to bf16), so
            // that the merged bits do not depend on which piece merges
            mp = mfin[rb];
            lp = lrow[rb];
#pragma unroll
            for (int db = 0; db < NO; ++db)
#pragma unroll
              for (int i = 0; i < 4; ++i)
                xo[db][i] = __uint_as_float(static_cast<uint32_t>(f32_to_bf16_rne(o[rb][db][i])) << 16);
          } else {
            const char *base = slot_ptr(pp);
            const float2 ml = reinterpret_cast<const float2 *>(base + C::PART_O)[wave * 32 + 16 * rb + l16];
            mp = ml.x;
            lp = ml.y;
            const uint2 *pO = reinterpret_cast<const uint2 *>(base);
#pragma unroll
            for (int db = 0; db < NO; ++db) {
              const uint2 x = pO[((wave * RB + rb) * NO + db) * kWave + l];
              xo[db] = f32x4{__uint_as_float(x.x << 16), __uint_as_float(x.x & 0xffff0000u),
                             __uint_as_float(x.y << 16), __uint_as_float(x.y & 0xffff0000u)};
            }
          }
          const float f = exp2f(mp - Mu);
          if (first) {
            first = false;
#pragma unroll
            for (int db = 0; db < NO; ++db)
#pragma unroll
              for (int i = 0; i < 4; ++i) acc[db][i] = xo[db][i] * f;
            lacc = lp * f;
          } else {
#pragma unroll
            for (int db = 0; db < NO; ++db)
#pragma unroll
              for (int i = 0; i < 4; ++i) acc[db][i] = fmaf(xo[db][i], f, acc[db][i]);   // one chain in piece order
            lacc = fmaf(lp, f, lacc);
          }
        }
#pragma unroll
        for (int db = 0; db < NO; ++db) o[rb][db] = acc[db];
        lrow[rb] = s_ok ? lacc : __builtin_nanf("");
        mfin[rb] = Mu;
      }
    }
  }

  if (emit) {
    // ---- normalise and store: o[rb][db][i] is row 32*wave + 16*rb + l16 at
    // d = 16*db + 4*g4 + i
  #pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int r = m_row0 + 32 * wave + 16 * rb + l16;
      const int node = r / G, g = r % G;
      if (node >= N) continue;
      const float fac = lrow[rb] > 0.f ? 1.0f / lrow[rb] : (lrow[rb] == 0.f ? 0.f : lrow[rb]);
      uint16_t *op = out + ((static_cast<int64_t>(m_b) * N + node) * Hq + m_kvh * G + g) * D + 4 * g4;
  #pragma unroll
      for (int db = 0; db < NO; ++db) {
        const uint32_t w0 = f32_to_bf16_rne(o[rb][db][0] * fac) |
                            (static_cast<uint32_t>(f32_to_bf16_rne(o[rb][db][1] * fac)) << 16);
        const uint32_t w1 = f32_to_bf16_rne(o[rb][db][2] * fac) |
                            (static_cast<uint32_t>(f32_to_bf16_rne(o[rb][db][3] * fac)) << 16);
        *reinterpret_cast<uint2 *>(op + 16 * db) = make_uint2(w0, w1);
      }
      if (lse && g4 == 0)
        lse[(static_cast<int64_t>(m_b) * N + node) * Hq + m_kvh * G + g] =
            lrow[rb] > 0.f ? (mfin[rb] + log2f(lrow[rb])) * 0.69314718055994531f
                           : (lrow[rb] == 0.f ? -INFINITY : lrow[rb]);
    }
  }
  __syncthreads();                       // the next piece reuses the LDS rings, mask and page ids
  };
  // A range holds one to three pieces at the workloads' shapes: those run as
  // straight-line copies of the piece (a loop around the key loop makes the
  // compiler keep values live across it and spill); more pieces loop.
  if (cur < my_hi) piece();
  if (cur < my_hi) piece();
  if (cur < my_hi) piece();
  while (cur < my_hi) piece();
}

template <int D, bool BIG>
int32_t launch_wide(int64_t blocks, hipStream_t st, const sdv_attn_shape &sh, int pshift, float scale_log2, int nrb,
                    int nwg, const uint16_t *q, const uint16_t *k_pool, const uint16_t *v_pool,
                    const int32_t *page_table, const int32_t *prefix_len, const uint32_t *mask_bits, uint16_t *out,
                    float *lse, unsigned *sync, char *parts, unsigned *status) {
  const size_t lds = WideCfg<D>::SMEM;
  static thread_local int configured_dev = -1;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(SDV_E_HIP, "tree_verify_attention: no device");
  if (configured_dev != dev) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(tree_attn_wide_kernel<D, BIG>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return fail(SDV_E_HIP, "tree_verify_attention: LDS attribute: %s", hipGetErrorString(e));
    configured_dev = dev;
  }
  hipLaunchKernelGGL((tree_attn_wide_kernel<D, BIG>), dim3(static_cast<unsigned>(blocks)), dim3(kAttnThreads), lds, st,
                     sh.B, sh.N, sh.Hq, sh.Hkv, pshift, sh.max_pages, sh.num_slots, scale_log2, nrb, nwg,
                     q, k_pool, v_pool, page_table, prefix_len, mask_bits, out, lse, sync, parts, status,
                     wait_limit(kMergeSpin));
  return check_launch("tree_attn_wide_kernel");
}

// Workgroups of the persistent schedule: the device's compute units, a
// multiple of the XCD count.
int persistent_workgroups() {
  const int n = num_cus() / kXcds * kXcds;
  return n >= kXcds ? n : kXcds;
}

}  // namespace

size_t attn_wide_workspace(int64_t units, int D) {
  if (2 * units > kAttnSyncWords) return 0;          // the persistent schedule is not offered for this many units
  Carver c(nullptr);
  c.take<char>(kWsHeaderBytes);
  c.take<unsigned>(kAttnSyncWords);
  c.take<char>(static_cast<size_t>(2 * persistent_workgroups()) * (D == 64 ? WideCfg<64>::PART : WideCfg<128>::PART));
  return c.bytes();
}

int32_t launch_attn_wide(hipStream_t st, const sdv_attn_shape &sh, int pshift, float scale_log2, int nrb, bool split,
                         const uint16_t *q, const uint16_t *k_pool, const uint16_t *v_pool,
                         const int32_t *page_table, const int32_t *prefix_len, const uint32_t *mask_bits,
                         uint16_t *out, float *lse, void *ws) {
  const int64_t units = static_cast<int64_t>(sh.B) * sh.Hkv;
  // the persistent schedule keeps every weighted position below 2^31
  const int64_t max_tiles = (static_cast<int64_t>(sh.max_pages) * sh.page + kTile - 1) / kTile;
  const bool persistent = split && sh.B <= kRankMax && persistent_workgroups() <= kMaxRanges &&
                          units * nrb * (kPieceWeight + kTileWeight * max_tiles) < (1LL << 31);
  const int nwg = persistent ? persistent_workgroups() : 0;
  const int64_t units_pad = (units + kXcds - 1) / kXcds * kXcds;
  const int64_t blocks = persistent ? nwg : units_pad * nrb;
  SDV_REQUIRE(blocks < (1LL << 31), SDV_E_UNSUPPORTED, "tree_verify_attention: grid too large");
  unsigned *sync = nullptr, *status = nullptr;
  char *parts = nullptr;
  if (persistent) {
    Carver c(ws);
    status = reinterpret_cast<unsigned *>(c.take<char>(kWsHeaderBytes)) + kWsStatus;
    sync = c.take<unsigned>(kAttnSyncWords);
    parts = c.take<char>(static_cast<size_t>(2 * nwg) * (sh.D == 64 ? WideCfg<64>::PART : WideCfg<128>::PART));
  }
  const bool big = static_cast<uint64_t>(sh.num_slots) * sh.Hkv * sh.D * 2 >= (1ull << 32);
#define SDV_WIDE(DD, BB)                                                                                       \
  launch_wide<DD, BB>(blocks, st, sh, pshift, scale_log2, nrb, nwg, q, k_pool, v_pool, page_table, prefix_len, \
                      mask_bits, out, lse, sync, parts, status)
  if (sh.D == 64) return big ? SDV_WIDE(64, true) : SDV_WIDE(64, false);
  return big ? SDV_WIDE(128, true) : SDV_WIDE(128, false);
#undef SDV_WIDE
}

}  // namespace sdv
