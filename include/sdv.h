/*
 * sdv.h -- C ABI of the MI355X (gfx950) library for the draft-tree build and
 * target-side verify step of EAGLE-style speculative decoding.
 *
 * Conventions for every entry point
 * ---------------------------------
 * - Pointers named "device" point to HIP device memory; pointers named "host"
 *   to host memory.  The caller owns every buffer; the library never frees
 *   caller memory and allocates nothing on these calls.  Scratch memory comes
 *   from a caller buffer `ws` of at least the bytes the matching
 *   `*_workspace_size` reports (NULL allowed when that size is 0).
 * - Every call is asynchronous on `stream` (a hipStream_t; NULL = the null
 *   stream) and performs no host synchronisation.  Outputs are valid once
 *   the stream reaches the call.  Calls are thread-safe; calls that share a
 *   workspace must not overlap on different streams.
 * - Arrays are dense, row-major, with the shapes given in brackets.  Token
 *   ids, positions, tree indices, slots and pages are int32.  bf16 values are
 *   passed as their raw 16-bit patterns (uint16_t).
 * - Inputs never alias outputs, except the documented in/out buffers of
 *   sdv_compact_kv.
 * - Return value: SDV_OK, or a negative status.  On error nothing has been
 *   enqueued, and sdv_last_error() returns a message for the calling thread.
 *   Shape checks run on the host; the kernels additionally clamp or skip
 *   out-of-range indices read from device arrays instead of faulting (the
 *   results of such inputs are unspecified).
 * - Device-side status: a workspace whose kernels wait on one another
 *   (sdv_draft_topk*, sdv_tree_verify_attention, sdv_verify_accept) or that
 *   carries a map between calls (sdv_tli_q_scatter) begins with a 256-byte
 *   header.  Its first 32-bit word is a sticky set of SDV_STATUS_* bits
 *   that a kernel sets when a bounded wait gave up (the outputs of that
 *   call are then unspecified) or when it met an input it could not use.
 *   sdv_workspace_status() reads it after the stream drains.
 *
 * Notation: B requests, k = topk, S = draft steps, N = tree size (root
 * included), V vocabulary, R = 1 + (S-1)*k draft-distribution rows per
 * request, M = k + (S-1)*k*k candidates per request.
 */
#ifndef SDV_H
#define SDV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  SDV_OK = 0,
  SDV_E_NULL = -1,        /* a required pointer is NULL */
  SDV_E_SHAPE = -2,       /* inconsistent shape (e.g. N-1 > M, Hq % Hkv != 0, k > V) */
  SDV_E_UNSUPPORTED = -3, /* a size outside what the kernels implement */
  SDV_E_WORKSPACE = -4,   /* workspace missing or too small */
  SDV_E_HIP = -5          /* the HIP runtime reported an error */
};

enum { SDV_ACCEPT_GREEDY = 0, SDV_ACCEPT_STOCHASTIC = 1 };

/* Message describing the last error of the calling thread ("" if none). */
const char *sdv_last_error(void);

/* ABI version (major * 100 + minor). */
int32_t sdv_version(void);

/* Device status bits (workspace header word 0). */
enum {
  SDV_STATUS_ACCEPT_WAIT = 1,      /* sdv_verify_accept: an exchange between the workgroups of a
                                      request gave up (a workgroup of the group was not running) */
  SDV_STATUS_ATTN_MERGE_WAIT = 2,  /* sdv_tree_verify_attention: the key split's merge gave up
                                      (the rows of that unit are NaN) */
  SDV_STATUS_TOPK_MERGE_WAIT = 4,  /* sdv_draft_topk*: a cut row's pieces did not all arrive (the
                                      row reads NaN / -1) */
  SDV_STATUS_TLI_REUSE = 8         /* sdv_tli_q_scatter: a call without ids found no map of its
                                      K and V_target in the workspace (its output is 0) */
};

/* Reads the status word of a workspace (device, ws_bytes as passed to the
 * call that used it; NULL or fewer than 256 bytes: status 0) into *status
 * (host) after draining `stream`, so the word reflects every call enqueued
 * before.  reset != 0 and a non-zero status: the whole workspace is then
 * zero-filled on `stream`, which restores the state the calls expect (a
 * wait that gave up may leave counters or exchange words behind) and clears
 * the status; the TLI scatter's map must then be built again.
 * The callers are error checks outside the hot loop: this call synchronises. */
int32_t sdv_workspace_status(void *ws, size_t ws_bytes, uint32_t *status, int32_t reset, void *stream);

/* Bounded waits between workgroups (the accept walk's exchanges, the
 * attention merge, the top-k piece merge) poll at most a library-chosen
 * number of times.  polls != 0xFFFFFFFF replaces that number for every call
 * enqueued afterwards (0: every such wait gives up at once, without
 * polling, so tests can drive the give-up paths while every kernel still
 * exits normally); 0xFFFFFFFF restores the library's choice.  Returns the
 * previous setting.  Process-wide; meant for tests. */
uint32_t sdv_set_wait_limit(uint32_t polls);

/* TLI shape validation.  sglang PR #22883, "Modified files": the TLI
 * validation block of the server-argument checks requires topk == 1 (TLI
 * does not support multi-candidate trees) and num_draft_tokens ==
 * num_steps + 1.  Returns SDV_OK, or SDV_E_UNSUPPORTED with a message.
 * Host only; a TLI pipeline calls it before its first step. */
int32_t sdv_tli_check(int32_t topk, int32_t num_steps, int32_t num_draft_tokens);

/* ------------------------------------------------------------------------
 * A1  Draft vocabulary top-k.
 * "[SGLang] Multi-Layer EAGLE", section 3 (draft extend): the per-step softmax
 * is reduced by fast_topk(probs, topk) to topk_p / topk_index.
 *
 * For every row r of probs (device, [rows, V] fp32, no NaN) writes the k
 * largest values in descending order to topk_p (device, [rows, k] fp32) and
 * their column ids to topk_id (device, [rows, k] int32).  Equal values are
 * ordered by ascending id.  1 <= k <= 32, k <= V, V < 2^31.
 *
 * Workspace (device, the size query's bytes; 0 when the rows are a multiple
 * of the device's compute units, or short): with rows = q * CUs + r, the
 * first q * CUs rows are scanned one workgroup each, and the r others are
 * cut into equal pieces spread over the compute units; a cut row is merged
 * by the workgroup that finishes it last, through per-row counters at the
 * start of the workspace (after the status header).  The caller
 * zero-fills the workspace once before its first use; every call leaves the
 * counters at zero again, so the same workspace serves later calls of any
 * shape.  Calls that share a workspace must not run concurrently.  Results
 * do not depend on the split (the k best under the order above are unique).
 * A merge that gives up sets SDV_STATUS_TOPK_MERGE_WAIT.
 * ---------------------------------------------------------------------- */
size_t sdv_draft_topk_workspace_size(int64_t rows, int32_t V, int32_t k);
int32_t sdv_draft_topk(const float *probs, int64_t rows, int32_t V, int32_t k,
                       float *topk_p, int32_t *topk_id, void *ws, size_t ws_bytes,
                       void *stream);

/* ------------------------------------------------------------------------
 * A1, fused from logits: the per-step softmax and fast_topk of the draft in
 * one pass ("[SGLang] Multi-Layer EAGLE", section 3: softmax then fast_topk
 * after each draft pass; the processed draft distribution is
 * softmax(logits / T)).  The probability rows are never materialised.
 *
 * For every row r of logits (device, [rows, V], dtype SDV_DTYPE_F32 or
 * SDV_DTYPE_BF16; entries may be -inf, at least one finite per row, no NaN)
 * writes to topk_p (device, [rows, k] fp32) the k largest values of
 * p = softmax(logits[r] / temperature), in descending order, and to topk_id
 * (device, [rows, k] int32) their column ids.  The order is that of the
 * exact probabilities, i.e. of the logits, lower id first among equal
 * logits (fp32 rounding of p never reorders).  p is computed in fp32 with
 * the row's normaliser accumulated in a fixed order (deterministic).
 * temperature > 0; 1 <= k <= 32, k <= V, V < 2^31.  Workspace: as for
 * sdv_draft_topk (zero-filled once, left zero-filled by every call); the
 * segments' normalisers are merged in segment order, so the values are
 * deterministic for a given device and shape.
 * ---------------------------------------------------------------------- */
enum { SDV_DTYPE_F32 = 0, SDV_DTYPE_BF16 = 1 };

size_t sdv_draft_topk_logits_workspace_size(int64_t rows, int32_t V, int32_t k);
int32_t sdv_draft_topk_logits(const void *logits, int32_t dtype, int64_t rows, int32_t V, int32_t k,
                              float temperature, float *topk_p, int32_t *topk_id, void *ws,
                              size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------
 * Processed distributions from logits: p = softmax(logits / T) per row, the
 * target-side processing the stochastic verify consumes and the draft's
 * per-step softmax ("[SGLang] Multi-Layer EAGLE", section 3: softmax, then
 * fast_topk, after each draft pass; zero-to-sglang ch.10 section 5.1: the
 * acceptance test compares the target's and the draft's probabilities).
 *
 * For every row r of logits (device, [rows, V] fp32, rows contiguous;
 * entries may be -inf, at least one finite per row, no NaN) writes
 * probs[r] (device, [rows, V] fp32) = exp((x - m) / T) / (sum of the same
 * over the row), m the row maximum.  Computed in fp32 as
 * 2^(x * c - m * c) with c = log2(e) / T and the normaliser summed in a
 * fixed order, so the result is deterministic for a given shape and
 * device; per entry within 3e-5 of the exact value, relative, for rows whose
 * finite logits span at most 64 * T.  A -inf entry gives exactly 0.
 * temperature finite and > 0; V >= 1; rows < 2^31.  probs must not alias
 * logits.  No workspace; asynchronous on `stream`.  Errors: SDV_E_SHAPE,
 * SDV_E_NULL, SDV_E_UNSUPPORTED, SDV_E_HIP.
 * ---------------------------------------------------------------------- */
int32_t sdv_softmax_rows(const float *logits, int64_t rows, int32_t V, float temperature, float *probs,
                         void *stream);

/* ------------------------------------------------------------------------
 * A2-A4  Candidate tree, positions, mask and retrieve arrays.
 * "[SGLang] Multi-Layer EAGLE", section 2 (select_top_k_tokens builds
 * tree_info = scores, tokens, parents with cumulative scores);
 * "EAGLE speculative decoding in four parts", "Drafting, verification and
 * slots" (build_eagle_tree expands the candidates into a tree and produces
 * the attention mask and positions) and "Exercises" (topk*S expansions plus
 * the root); zero-to-sglang ch.10 section 5.2 (verify input: draft tokens,
 * positions, custom mask, retrieve arrays).
 *
 * Inputs (device): topk_p / topk_id [B, R, k] -- row 0 is the root's top-k,
 * row 1 + i*k + j the top-k after frontier slot j of draft step i;
 * root_token [B]; prefix_len [B] (tokens whose KV is cached).
 * Step 0 pools the root's k children (score = prob).  Step i >= 1 pools the k
 * children of every frontier slot j (score = fp32 product parent*prob, pool
 * index = step, slot, child rank); the next frontier is the best k of them.
 * The tree is node 0 = root plus the best N-1 pool entries (score desc, pool
 * index asc) in ascending pool index.  topk_p must lie in [0, 1].
 * Outputs (device, [B, N] unless noted):
 *   tokens, parent (-1 for the root), depth, positions = prefix_len + depth,
 *   score (fp32, root 1.0), q_row (draft row of the node's children; -1 if
 *   the node was never expanded; 0 for the root),
 *   mask [B, N, N] uint8 (1 iff column j is the row's node or an ancestor;
 *   NULL to skip), mask_bits [B, N, ceil(N/32)] uint32 (bit j%32 of word j/32;
 *   NULL to skip), retrieve_index (b*N + i), retrieve_next_token (smallest
 *   child or -1), retrieve_next_sibling (next larger sibling or -1).
 * Limits: 1 <= k <= 32, S >= 1, 1 <= N <= min(M + 1, 256), M <= 2048.
 * ---------------------------------------------------------------------- */
typedef struct {
  int32_t B, k, S, N;
} sdv_tree_shape;

int32_t sdv_build_tree(sdv_tree_shape shape, const float *topk_p, const int32_t *topk_id,
                       const int32_t *root_token, const int32_t *prefix_len, int32_t *tokens,
                       int32_t *parent, int32_t *depth, int32_t *positions, float *score,
                       int32_t *q_row, uint8_t *mask, uint32_t *mask_bits,
                       int32_t *retrieve_index, int32_t *retrieve_next_token,
                       int32_t *retrieve_next_sibling, void *stream);

/* ------------------------------------------------------------------------
 * Multi-layer draft chain.  "[SGLang] Multi-Layer EAGLE", sections 2-3:
 * each draft step runs its own layer and takes its top-k; the per-step
 * lists are concatenated along the step dimension, and the draft slices them
 * by step -- step i gives one node whose parent is the node of step i-1 (the
 * root for step 0) and whose score is step i's own probability.
 *
 * Inputs (device): topk_p / topk_id [B, S] (each step's top-1; the tree
 * layout [B, S, 1] is the same memory), root_token [B], prefix_len [B].
 * Outputs as sdv_build_tree with N = S + 1: node i+1 = step i's token,
 * parent[i] = i - 1, depth = i, positions = prefix_len + i, score = 1.0 for
 * the root and topk_p[b, i-1] otherwise (not a product), q_row[i] = i
 * (the draft row of step i) and -1 for the last node, mask = the lower
 * triangle, retrieve_next_token[i] = i + 1 (-1 last), no siblings.
 * mask and mask_bits may be NULL.  Limits: 1 <= S <= 255.
 * ---------------------------------------------------------------------- */
int32_t sdv_build_chain(int32_t B, int32_t S, const float *topk_p, const int32_t *topk_id,
                        const int32_t *root_token, const int32_t *prefix_len, int32_t *tokens,
                        int32_t *parent, int32_t *depth, int32_t *positions, float *score,
                        int32_t *q_row, uint8_t *mask, uint32_t *mask_bits, int32_t *retrieve_index,
                        int32_t *retrieve_next_token, int32_t *retrieve_next_sibling, void *stream);

/* ------------------------------------------------------------------------
 * A5  Tree-verify attention.
 * "EAGLE speculative decoding in four parts": verification is one target
 * forward over 1 + candidates tokens per request with a tree attention mask
 * ("Self-test" answer 1, "Exercises" question 1, "Design trade-offs");
 * "[SGLang] Multi-Layer EAGLE" section 6 (TARGET_VERIFY with the custom mask).
 *
 * For request b, node i, query head h: attends to every prefix key (logical
 * positions 0 .. prefix_len[b]-1) and to tree key j (logical position
 * prefix_len[b] + j) iff bit j of mask_bits[b, i] is set;
 * out = softmax(sm_scale * q.k) v over those keys, KV head h / (Hq/Hkv).
 * q: device [B, N, Hq, D] bf16.  k_pool, v_pool: device [num_slots, Hkv, D]
 * bf16 (token-major).  page_table: device [B, max_pages] int32; logical
 * position p lives in slot page_table[b][p / page] * page + p % page
 * (page == 1: a slot map).  prefix_len: device [B], with
 * prefix_len + N <= max_pages * page.  mask_bits: device [B, N, ceil(N/32)].
 * out: device [B, N, Hq, D] bf16; lse: device [B, N, Hq] fp32 natural-log
 * sum of exp(sm_scale * q.k) (NULL to skip).  sm_scale <= 0 selects
 * 1/sqrt(D).  Limits: D in {64, 128}, 1 <= N <= 256, Hq % Hkv == 0,
 * Hq/Hkv <= 16, page a power of two, 1 <= num_slots, num_slots + page < 2^31
 * and num_slots * Hkv * D * 2 < 2^36 bytes per pool.  A page id outside the
 * pool is an input error: no read leaves the pools and the outputs of the
 * rows that see such a key are unspecified.
 * Workspace: when N * Hq/Hkv > 128 (and B * Hkv * ceil(N * Hq/Hkv / 256) <=
 * 4096) the size query returns the bytes with which a call may split each
 * unit's keys over two workgroups (few units, many CUs).  ws must then be
 * 256-byte aligned and zero-filled once before its first use: after the
 * 256-byte status header, 32 KiB hold counters that every call leaves at
 * zero, whatever the shape, and the rest is scratch.  Calls that may overlap
 * need separate workspaces.  ws = NULL (or fewer bytes) runs without the
 * split.  A merge that gives up sets SDV_STATUS_ATTN_MERGE_WAIT.
 * Otherwise the size query returns 0 and ws is ignored.
 * ---------------------------------------------------------------------- */
typedef struct {
  int32_t B, N, Hq, Hkv, D, page, max_pages;
  int64_t num_slots;
} sdv_attn_shape;

size_t sdv_tree_verify_attention_workspace_size(sdv_attn_shape shape);
int32_t sdv_tree_verify_attention(sdv_attn_shape shape, float sm_scale, const uint16_t *q,
                                  const uint16_t *k_pool, const uint16_t *v_pool,
                                  const int32_t *page_table, const int32_t *prefix_len,
                                  const uint32_t *mask_bits, uint16_t *out, float *lse,
                                  void *ws, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------
 * A6-A7  Target row reductions and the accept walk.
 * zero-to-sglang ch.10: section 3.3 (row alignment: a node's target row
 * verifies its children; the last row picks the bonus), section 4.1
 * (greedy_commit: commit the target's choice, stop at the first mismatch, at
 * EOS or when the budget is used up; bonus after a full match), section 5.1
 * (accept y with probability min(1, p[y]/q[y]); on rejection draw from the
 * normalised positive residual; bonus from p); "EAGLE speculative decoding
 * in four parts", "Drafting, verification and slots" (the verification
 * kernels walk each request's tree to its longest accepted path).
 *
 * Tree inputs (device, [B, N]): tokens, next_token, next_sibling (as written
 * by sdv_build_tree), q_row (stochastic only).  target: device [B, N, V] fp32,
 * row u = the target after node u (GREEDY: logits; STOCHASTIC: processed
 * probabilities p).  draft_probs: device [B, R, V] fp32 processed draft
 * distributions (STOCHASTIC only; may be NULL for GREEDY).  u_accept, u_draw:
 * device [B, N] fp32 uniforms of the form kk * 2^-24 (STOCHASTIC only):
 * u_accept[b, c] decides child node c, u_draw[b, u] is the draw at node u.
 * eos_id: token that ends a request (-1: none).  remaining: device [B]
 * output budgets (NULL: unlimited).
 * Greedy: at node u take t = argmax(row u) (lowest id on ties), commit t,
 * stop on EOS or budget, move to the child carrying t or stop.
 * Stochastic: t := p_u; for the children in sibling order accept child c iff
 * double(u_accept) * double(q[y]) < double(t[y]); on rejection
 * r = max(t - q, 0) (fp32), masses floor(r * 2^40) (uint64, sum S), and
 * t := fp32(double(r) / (double(S) * 2^-40)) when S > 0.  All children
 * rejected: draw from the last residual's masses; leaf: draw from
 * floor(p * 2^40); draw T = floor(kk * S / 2^24), token = least i whose
 * running mass exceeds T; zero total mass: argmax of t.
 * Outputs (device): accept_len [B]; accept_path [B, S+1] (tree indices, root
 * first, -1 padded); commit_tokens [B, S+1] (-1 padded); commit_len [B];
 * next_root [B] (last committed token, -1 if none).
 * p and q entries lie in [0, 1] (rows need not sum to 1).
 * Limits: V < 2^31 - 4, N <= 256, S + 1 <= 64.  The W workgroups of a
 * request exchange row-wide values and must run at the same time: the
 * launch holds no more workgroups than the device keeps resident, and an
 * exchange that still misses a word after its bounded wait sets
 * SDV_STATUS_ACCEPT_WAIT (e.g. when other work occupies the device).  Calls
 * that share a workspace must not overlap.  The workspace must be
 * zero-filled before its first use; every call leaves it zero-filled
 * (whatever its shape), so one zero-filled buffer of the largest size
 * query's bytes serves every later call.
 * ---------------------------------------------------------------------- */
typedef struct {
  int32_t B, N, S, V, R, mode;
} sdv_accept_shape;

size_t sdv_verify_accept_workspace_size(sdv_accept_shape shape);
int32_t sdv_verify_accept(sdv_accept_shape shape, int32_t eos_id, const int32_t *remaining,
                          const int32_t *tokens, const int32_t *next_token,
                          const int32_t *next_sibling, const int32_t *q_row, const float *target,
                          const float *draft_probs, const float *u_accept, const float *u_draw,
                          int32_t *accept_len, int32_t *accept_path, int32_t *commit_tokens,
                          int32_t *commit_len, int32_t *next_root, void *ws, size_t ws_bytes,
                          void *stream);

/* ------------------------------------------------------------------------
 * The accept walk for callers that cannot allocate memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation).
 * Same arguments, semantics and outputs as sdv_verify_accept, without the
 * workspace: the exchange words of up to 1024 requests live in a static
 * device array of the library (1,052,928 bytes per device, held until the
 * process ends).  Each call zero-fills the part it uses with a kernel on
 * `stream` (no memset node) before the walk, so it calls no allocator and no
 * hipMemset.  B > 1024 returns SDV_E_UNSUPPORTED.  Every call on one device
 * shares that array: calls that may overlap on one device (different
 * streams, host threads) race and must be serialised by the caller.  The
 * status word of a wait that gave up is cleared by the next call; callers
 * that need it use sdv_verify_accept with their own workspace.
 * ---------------------------------------------------------------------- */
int32_t sdv_verify_accept_noalloc(sdv_accept_shape shape, int32_t eos_id, const int32_t *remaining,
                                  const int32_t *tokens, const int32_t *next_token,
                                  const int32_t *next_sibling, const int32_t *q_row, const float *target,
                                  const float *draft_probs, const float *u_accept, const float *u_draw,
                                  int32_t *accept_len, int32_t *accept_path, int32_t *commit_tokens,
                                  int32_t *commit_len, int32_t *next_root, void *stream);

/* ------------------------------------------------------------------------
 * A8  KV compaction of the accepted path and release of the rest.
 * "EAGLE speculative decoding in four parts": slots for every candidate are
 * reserved before drafting; after verification only the accepted path's
 * slots are kept and the rest freed, and with page size > 1 the last page is
 * copied ("Self-test" answer 3, "Drafting, verification and slots",
 * "Design trade-offs"); zero-to-sglang ch.10 section 5.2 (the cache returns
 * to the committed path; the correction or bonus token has no KV yet).
 *
 * Tree of request b: logical positions L .. L+N-1 (node j at L + j, L =
 * prefix_len[b]).  accept_len [B] = a, accept_path [B, S+1] = path (path[0]
 * = 0, strictly increasing, < N), both device.  Position L + d must end up
 * holding node path[d]'s KV, d = 0..a; new_len[b] = L + a + 1.
 * page == 1: page_table (device [B, max_pages], in/out) is a slot map;
 * entries L + d are remapped, L+a+1 .. L+N-1 set to -1, no KV bytes move,
 * and the rejected nodes' old slots are freed in ascending node order.
 * page > 1: the K and V rows [Hkv, D] of every layer are copied from
 * position L + path[d] to L + d (all reads of a request happen before its
 * writes); logical pages ceil(new_len/page) .. (L+N-1)/page are set to -1
 * in page_table and their page ids freed in page order.
 * k_pools, v_pools: HOST arrays of `layers` device pointers to
 * [num_slots, Hkv, D] bf16 pools (in/out; unused when page == 1).
 * freed: device [B*N] int32, the freed ids of all requests in batch order;
 * num_freed: device [1] int32.  new_len: device [B].
 * Workspace (page > 1): the size query's bytes (the moved tokens' slot
 * pairs), no initialisation needed; page == 1 needs none.
 * Limits: N <= 256, layers <= 128; page > 1 also S <= 63 and
 * (Hkv * D) % 8 == 0.
 * ---------------------------------------------------------------------- */
typedef struct {
  int32_t B, N, S, page, Hkv, D, layers, max_pages;
  int64_t num_slots;
} sdv_kv_shape;

size_t sdv_compact_kv_workspace_size(sdv_kv_shape shape);
int32_t sdv_compact_kv(sdv_kv_shape shape, uint16_t *const *k_pools, uint16_t *const *v_pools,
                       int32_t *page_table, const int32_t *prefix_len, const int32_t *accept_len,
                       const int32_t *accept_path, int32_t *new_len, int32_t *freed,
                       int32_t *num_freed, void *ws, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------
 * KV slot / page allocation around a speculative step.
 * "EAGLE speculative decoding in four parts", "Drafting, verification and
 * slots": with page size 1 the draft reserves batch x topk x steps slots at
 * once with the allocator's state backed up, rolled back after the step;
 * with page size > 1, topk = 1 extends each request's own sequence and
 * topk > 1 duplicates the last partial page, every branch holding a copy of
 * the prefix's partial page followed by its draft tokens; "Design
 * trade-offs": allocate first, roll back after.  "[SGLang] Multi-Layer
 * EAGLE" section 6: draft and target share one allocator.
 *
 * Units are slots (page == 1) or pages (page > 1).  Allocator (device,
 * caller-owned): free_ids [capacity] int32 and state [4] int32 = {top,
 * pushes, error, 0}; the free units are free_ids[0 .. top), free_ids[top-1]
 * is handed out first.  error is a sticky bit set: 1 no room (or a table
 * row would overflow), 2 restore refused, 4 release overflow, 8 corrupt
 * state, 16 partial-page slot outside the pool.  A failed call changes no
 * allocator or table entry (its position outputs read -1).
 *   init: free_ids = capacity-1 .. 0 (units come out ascending), top =
 *     capacity, pushes = error = 0.  A caller may instead fill free_ids
 *     with any distinct unit ids itself and set state = {count, 0, 0, 0}.
 *   backup: backup [2] (device) = {top, pushes}.
 *   restore: top = backup top, allowed only if nothing was released since
 *     the backup (pushes unchanged) and backup top >= top -- it undoes the
 *     allocations made since.
 *   free: pushes ids[0 .. *num_ids) (num_ids on the device, at most
 *     max_ids), e.g. sdv_compact_kv's freed list; pushes += 1.
 *   extend: request b of length L = seq_len[b] takes positions L .. L+n-1
 *     of its own chain, requests in batch order.  page == 1: page_table is a
 *     slot map [B, max_pages] and gets one slot per position; page > 1: the
 *     partial last page is continued and pages ceil(L/P) .. ceil((L+n)/P)-1
 *     are appended to the row.  out_loc [B, n] = slot of position L+i.
 *   branches: with r = L mod P, branch j of request b takes
 *     ceil((r + S) / P) pages of its own (requests, branches, pages in
 *     order): branch_pages [B, topk, sdv_kv_branch_pages(page, S)], -1
 *     padded; the K and V rows of the r partial-page positions (every layer,
 *     pools as in sdv_compact_kv) are copied into the first r slots of each
 *     branch; out_loc [B, topk, S] = slot of draft step i of branch j =
 *     branch_pages[b][j][(r+i)/P]*P + (r+i) mod P.  page == 1 gives one slot
 *     per (request, branch, step); page_table is read only; layers may be 0
 *     (no copy).
 * Limits: B <= 8192.  Calls on one allocator must be stream ordered.
 * ---------------------------------------------------------------------- */
typedef struct {
  int32_t B, page, topk, S, Hkv, D, layers, max_pages;
  int64_t num_slots;
} sdv_branch_shape;

int32_t sdv_kv_branch_pages(int32_t page, int32_t S);
int32_t sdv_kv_alloc_init(int32_t capacity, int32_t *free_ids, int32_t *state, void *stream);
int32_t sdv_kv_alloc_backup(const int32_t *state, int32_t *backup, void *stream);
int32_t sdv_kv_alloc_restore(int32_t capacity, int32_t *state, const int32_t *backup, void *stream);
int32_t sdv_kv_alloc_free(int32_t capacity, int32_t *free_ids, int32_t *state, const int32_t *ids,
                          const int32_t *num_ids, int32_t max_ids, void *stream);
int32_t sdv_kv_alloc_extend(int32_t capacity, int32_t *free_ids, int32_t *state, int32_t B, int32_t page,
                            int32_t n, int32_t *page_table, int32_t max_pages, const int32_t *seq_len,
                            int32_t *out_loc, void *stream);
int32_t sdv_kv_alloc_branches(int32_t capacity, int32_t *free_ids, int32_t *state, sdv_branch_shape shape,
                              uint16_t *const *k_pools, uint16_t *const *v_pools, const int32_t *page_table,
                              const int32_t *seq_len, int32_t *branch_pages, int32_t *out_loc, void *stream);

/* ------------------------------------------------------------------------
 * A9  TLI pruned draft LM head.
 * sglang PR #22883 "TLI (Token-Level Intersection)", "Modifications": the
 * draft LM head becomes a compact [intersection_size x hidden_dim] matrix,
 * turning the dominant draft matmul from O(B*V_draft*H) into O(B*K*H).
 *
 * logits[b, j] = sum_h hidden[b, h] * weight[j, h] with fp32 accumulation.
 * hidden: device [B, H] bf16; weight: device [K, H] bf16 (row j belongs to
 * draft id intersection_draft_ids[j]); logits: device [B, K] fp32.
 * Limits: H % 32 == 0, B >= 1, K >= 1.
 * ---------------------------------------------------------------------- */
int32_t sdv_tli_lm_head(int32_t B, int32_t H, int32_t K, const uint16_t *hidden,
                        const uint16_t *weight, float *logits, void *stream);

/* ------------------------------------------------------------------------
 * A10  TLI vocabulary maps, logit constraint and distribution scatter.
 * sglang PR #22883, "Modifications": constrain_draft_logits (logits outside
 * the intersection -> -inf), map_target_to_draft_ids,
 * map_draft_to_target_ids, sorted intersection_draft_ids, EOS fallback for
 * models without an unknown token; the target's rejection sampling is
 * unchanged.
 *
 * sdv_tli_build_maps: from K pairs (inter_ids[j] draft id, tgt_ids[j] target
 * id; device [K] each, in range, distinct) writes d2t (device [V_draft], -1
 * outside the intersection) and t2d (device [V_target], `fallback` outside).
 * sdv_tli_map_ids: out[i] = table[ids[i]] (device arrays; ids outside
 * [0, table_len) give -1) -- map_target_to_draft_ids with t2d,
 * map_draft_to_target_ids with d2t.
 * sdv_tli_constrain_draft_logits: full[b, inter_ids[j]] = pruned[b, j], -inf
 * elsewhere; pruned device [B, K] fp32, inter_ids device [K] sorted
 * ascending, full device [B, V_draft] fp32.
 * sdv_tli_q_scatter: q_target[r, tgt_ids[j]] = q_pruned[r, j], 0 elsewhere;
 * q_pruned device [rows, K] fp32, q_target device [rows, V_target] fp32;
 * the workspace holds a header (K and V_target of the map) and the inverse
 * of tgt_ids; a call with tgt_ids builds them (whatever
 * the workspace held, its status word included, is overwritten).  The
 * workspace needs no zero-fill.  tgt_ids == NULL reuses what an earlier
 * call with the same K and V_target left in the same workspace (the maps
 * are static, so a serving loop builds them once); if the header names
 * another K or V_target (or no map was built), the output is 0 and
 * SDV_STATUS_TLI_REUSE is set.  Ids and positions read from the workspace
 * are bounds-checked against K.  K == 0 writes zeros and leaves the
 * workspace as it was.
 * ---------------------------------------------------------------------- */
int32_t sdv_tli_build_maps(int32_t K, const int32_t *inter_ids, const int32_t *tgt_ids,
                           int32_t V_draft, int32_t V_target, int32_t fallback, int32_t *d2t,
                           int32_t *t2d, void *stream);
int32_t sdv_tli_map_ids(const int32_t *table, int32_t table_len, const int32_t *ids, int64_t n,
                        int32_t *out, void *stream);
int32_t sdv_tli_constrain_draft_logits(int32_t B, int32_t K, int32_t V_draft, const float *pruned,
                                       const int32_t *inter_ids, float *full, void *stream);
size_t sdv_tli_q_scatter_workspace_size(int32_t V_target);
int32_t sdv_tli_q_scatter(int64_t rows, int32_t K, int32_t V_target, const float *q_pruned,
                          const int32_t *tgt_ids, float *q_target, void *ws, size_t ws_bytes,
                          void *stream);

/* ------------------------------------------------------------------------
 * Draft extend after a verify step: index preparation.
 * "EAGLE speculative decoding in four parts", "Self-test" answer 1 (after
 * verification the draft model runs one extend over the accepted tokens to
 * prepare the next round); zero-to-sglang ch.10 section 3.1 (draft, verify,
 * then the draft-side extend for the next round); sglang PR #22883
 * "Modifications" (under TLI the accepted tokens are mapped target -> draft
 * for that extend; the target ids themselves are left as they are).
 *
 * Inputs, as sdv_verify_accept writes them (device): commit_len [B],
 * commit_tokens [B, S+1], accept_path [B, S+1]; prefix_len [B] as given to
 * the tree build.  Committed token j of request b was chosen at node
 * accept_path[b, j].  t2d: device [V_target] target -> draft map (as
 * sdv_tli_build_maps writes it), or NULL for no mapping.
 * Outputs (device, int32), requests packed in batch order:
 *   extend_start [B+1]: extend_start[b] = sum of commit_len over requests
 *     before b; extend_start[B] = total rows;
 *   for row = extend_start[b] + j, j < commit_len[b]:
 *     input_ids[row]    = commit_tokens[b, j], through t2d when given;
 *     positions[row]    = prefix_len[b] + 1 + j;
 *     hidden_index[row] = b * N + accept_path[b, j] (the verify output row
 *                         of the node that chose the token);
 *   last_index [B] = extend_start[b] + commit_len[b] - 1 (-1 if none);
 *   seq_len [B] = prefix_len[b] + 1 + commit_len[b].
 * input_ids, positions, hidden_index need room for B * (S+1) rows; rows past
 * the total are not written.  A commit_len outside [0, S+1] is clamped into
 * it; a negative token, or one outside [0, V_target) when t2d is given,
 * gives input_id -1, and a node outside [0, N) gives hidden_index -1.
 * Limits: B * N < 2^31.
 * ---------------------------------------------------------------------- */
int32_t sdv_draft_extend_prep(int32_t B, int32_t N, int32_t S, const int32_t *prefix_len,
                              const int32_t *commit_len, const int32_t *commit_tokens,
                              const int32_t *accept_path, const int32_t *t2d, int32_t V_target,
                              int32_t *extend_start, int32_t *input_ids, int32_t *positions,
                              int32_t *hidden_index, int32_t *last_index, int32_t *seq_len,
                              void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SDV_H */
