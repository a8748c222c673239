"""Oracle: candidate tree from the per-step draft top-k, and its verify arrays.

Follows
* "[SGLang] Multi-Layer EAGLE", section 2 (draft step): ``select_top_k_tokens``
  turns each step's ``topk_p`` / ``topk_index`` into ``tree_info`` = (scores,
  tokens, parents), scores accumulating along the path;
* "EAGLE speculative decoding in four parts", "Drafting, verification and
  slots": ``build_eagle_tree`` expands the candidates into a tree and produces
  the attention mask and positions for verification; "Exercises", question 1:
  with num_steps=3, topk=4 the draft expands 4+4+4 frontier candidates plus the
  root;
* zero-to-sglang ch.10, section 5.2: the verify input carries the draft tokens,
  their positions, the custom mask and the retrieve arrays.

Readings where the pages leave a step open:
1. Pool.  Step 0 puts the root's k children in the pool with score = prob.
   Each later step expands every frontier slot j of the previous step into its
   k children with score = fl32(score(parent) * prob); all of them join the
   pool (k + (S-1)*k*k entries) and the new frontier is the best k of them.
   The final tree is the best N-1 entries of the whole pool.
2. Scores are fp32 products taken in root-to-node order (root score 1.0).
3. "Best" orders by score descending, then pool index ascending; pool index
   runs over (step, frontier slot, child rank).
4. Frontier slot j of step i is the j-th best entry of that step; the
   distribution of its children is draft row 1 + i*k + j (row 0 is the root's).
5. Tree node 0 is the root; nodes 1..N-1 are the selected pool entries in
   ascending pool index, so parents precede children and siblings keep their
   child-rank order.
6. positions = prefix_len + depth, prefix_len counting the tokens whose KV is
   already cached (the root is the last committed token, which has none yet).
7. The mask covers the tree only ([N, N]); the prefix is visible to every node.
8. retrieve_index[i] = b*N + i; next_token[i] = the smallest-index child or -1;
   next_sibling[i] = the next larger-index child of the same parent or -1.
"""
from __future__ import annotations

from typing import Dict, List

import numpy as np


class TreeBuilder:
    """Step-wise EAGLE-2 style tree construction for one request.

    ``start`` consumes the root's top-k; every ``expand`` consumes the top-k
    rows of the current frontier (slot order) and adds one draft step.  The
    step-wise form lets a test drive the draft model node by node.
    """

    def __init__(self, k: int, S: int):
        if k < 1 or S < 1:
            raise ValueError("need k >= 1 and S >= 1")
        self.k, self.S = k, S
        self.score: List[np.float32] = []
        self.token: List[int] = []
        self.parent: List[int] = []       # pool index of the parent, -1 = root
        self.step: List[int] = []
        self.row_of: Dict[int, int] = {}  # pool index -> draft row of its children
        self.frontier: List[int] = []
        self.steps_done = 0

    def _best(self, idxs, n):
        return sorted(idxs, key=lambda e: (-float(self.score[e]), e))[:n]

    def start(self, p_row, id_row):
        """Draft step 0: the root's top-k become the first candidates."""
        assert self.steps_done == 0
        for c in range(self.k):
            self.score.append(np.float32(p_row[c]))
            self.token.append(int(id_row[c]))
            self.parent.append(-1)
            self.step.append(0)
        self.frontier = self._best(range(self.k), self.k)
        self.steps_done = 1

    def frontier_rows(self):
        """Draft row index that the frontier slot j's children come from."""
        i = self.steps_done - 1
        return [1 + i * self.k + j for j in range(len(self.frontier))]

    def expand(self, p_rows, id_rows):
        """One further draft step: p_rows[j], id_rows[j] are the top-k of the
        distribution after frontier slot j."""
        assert 1 <= self.steps_done < self.S
        i = self.steps_done
        rows = self.frontier_rows()
        new = []
        for j, f in enumerate(self.frontier):
            self.row_of[f] = rows[j]
            for c in range(self.k):
                s = np.float32(self.score[f]) * np.float32(p_rows[j][c])
                new.append(len(self.score))
                self.score.append(np.float32(s))
                self.token.append(int(id_rows[j][c]))
                self.parent.append(f)
                self.step.append(i)
        self.frontier = self._best(new, self.k)
        self.steps_done += 1

    def path_tokens(self, e):
        """Tokens from the first draft step down to pool entry ``e``."""
        out = []
        while e >= 0:
            out.append(self.token[e])
            e = self.parent[e]
        return out[::-1]

    def finalize(self, N: int, root_token: int, prefix_len: int, b: int = 0):
        assert self.steps_done == self.S
        M = len(self.score)
        if not 1 <= N <= M + 1:
            raise ValueError("need 1 <= N <= 1 + pool size")
        chosen = sorted(self._best(range(M), N - 1))
        tree_of = {e: t + 1 for t, e in enumerate(chosen)}
        tokens = np.empty(N, np.int32)
        parent = np.empty(N, np.int32)
        depth = np.empty(N, np.int32)
        score = np.empty(N, np.float32)
        q_row = np.empty(N, np.int32)
        tokens[0], parent[0], depth[0], score[0], q_row[0] = root_token, -1, 0, 1.0, 0
        for e in chosen:
            t = tree_of[e]
            pe = self.parent[e]
            if pe >= 0 and pe not in tree_of:
                raise ValueError("selected node's parent not selected (probabilities above 1?)")
            tokens[t] = self.token[e]
            parent[t] = 0 if pe < 0 else tree_of[pe]
            depth[t] = self.step[e] + 1
            score[t] = self.score[e]
            q_row[t] = self.row_of.get(e, -1)
        return verify_arrays(tokens, parent, depth, score, q_row, prefix_len, b)


def verify_arrays(tokens, parent, depth, score, q_row, prefix_len, b):
    """Mask, positions and retrieve arrays of one request's tree."""
    N = tokens.shape[0]
    W = (N + 31) // 32
    mask = np.zeros((N, N), np.uint8)
    for i in range(N):
        j = i
        while j >= 0:
            mask[i, j] = 1
            j = int(parent[j])
    bits = np.zeros((N, W), np.uint32)
    for i in range(N):
        for j in range(N):
            if mask[i, j]:
                bits[i, j // 32] |= np.uint32(1 << (j % 32))
    next_token = np.full(N, -1, np.int32)
    next_sibling = np.full(N, -1, np.int32)
    for i in range(1, N):
        p = int(parent[i])
        if next_token[p] < 0:
            next_token[p] = i
        for j in range(i + 1, N):
            if parent[j] == p:
                next_sibling[i] = j
                break
    return dict(
        tokens=tokens, parent=parent, depth=depth, score=score, q_row=q_row,
        positions=(depth + np.int32(prefix_len)).astype(np.int32),
        mask=mask, mask_bits=bits,
        retrieve_index=(np.arange(N, dtype=np.int32) + np.int32(b * N)),
        next_token=next_token, next_sibling=next_sibling,
    )


def build_tree(topk_p, topk_id, root_token, prefix_len, k: int, S: int, N: int):
    """Batched tree build from precomputed top-k rows.

    ``topk_p`` / ``topk_id``: [B, R, k] with R = 1 + (S-1)*k (row 0 the root's,
    row 1 + i*k + j the children of frontier slot j of step i).
    Returns a dict of [B, N] (and [B, N, N], [B, N, ceil(N/32)]) arrays.
    """
    topk_p = np.asarray(topk_p, np.float32)
    topk_id = np.asarray(topk_id, np.int32)
    B, R, kk = topk_p.shape
    if kk != k or R != 1 + (S - 1) * k:
        raise ValueError("top-k rows do not match (k, S)")
    per = []
    for b in range(B):
        tb = TreeBuilder(k, S)
        tb.start(topk_p[b, 0], topk_id[b, 0])
        for _ in range(1, S):
            rows = tb.frontier_rows()
            tb.expand([topk_p[b, r] for r in rows], [topk_id[b, r] for r in rows])
        per.append(tb.finalize(N, int(root_token[b]), int(prefix_len[b]), b))
    return {key: np.stack([d[key] for d in per]) for key in per[0]}


def build_chain(topk_p, topk_id, root_token, prefix_len):
    """Multi-layer (MTP) draft chain: one token per draft step.

    "[SGLang] Multi-Layer EAGLE", sections 2-3: each step runs its own draft
    layer and takes its top-k; the per-step lists are concatenated along the
    step dimension, and with several steps the draft slices ``tree_info`` by
    step: step i contributes the score and token of column i, step 0's parent
    is the root and step i's parent is index i, the token of the step before.
    The tree is the chain root -> step 0 -> ... -> step S-1 (N = S + 1 nodes)
    and each node keeps its own step's score (no product along the path).

    ``topk_p`` / ``topk_id``: [B, S] (or [B, S, 1]) top-1 of each step.
    Readings: node i+1 is step i's token; its children come from draft row
    i + 1 (the next step), the last node is never expanded (q_row -1), the
    root's children come from row 0; positions, mask and retrieve arrays as for
    the tree (``verify_arrays``).  Returns the same keys as ``build_tree``.
    """
    topk_p = np.asarray(topk_p, np.float32)
    topk_id = np.asarray(topk_id, np.int32)
    if topk_p.ndim == 3:
        if topk_p.shape[2] != 1:
            raise ValueError("a chain takes one token per step")
        topk_p, topk_id = topk_p[:, :, 0], topk_id[:, :, 0]
    B, S = topk_p.shape
    if S < 1:
        raise ValueError("need S >= 1")
    N = S + 1
    per = []
    for b in range(B):
        tokens = np.array([int(root_token[b])] + [int(x) for x in topk_id[b]], np.int32)
        parent = np.array([-1] + list(range(S)), np.int32)
        depth = np.arange(N, dtype=np.int32)
        score = np.array([1.0] + [float(x) for x in topk_p[b]], np.float32)
        q_row = np.array(list(range(S)) + [-1], np.int32)
        per.append(verify_arrays(tokens, parent, depth, score, q_row, int(prefix_len[b]), b))
    return {key: np.stack([d[key] for d in per]) for key in per[0]}
