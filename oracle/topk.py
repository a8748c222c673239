"""Oracle: per-row top-k of the draft distributions.

Follows "[SGLang] Multi-Layer EAGLE", section 3 (draft extend): after each
draft pass the per-row softmax is reduced by ``fast_topk(probs, topk)`` to the
``topk_p`` / ``topk_index`` pairs that feed the tree.  The pages fix no tie
rule; a fixed one is required for greedy verification to reproduce target-only
decoding (zero-to-sglang ch.10, section 4.2), so ties go to the lower token id.

Definition: the k entries that come first when the row is ordered by
probability descending, then token id ascending; returned in that order.
"""
from __future__ import annotations

import numpy as np


def draft_topk(probs: np.ndarray, k: int):
    """Top-k of every row of ``probs`` ([..., V] fp32).

    Returns ``(topk_p [..., k] fp32, topk_id [..., k] int32)``.  Rows must hold
    no NaN.  Ties: lower id first.
    """
    p = np.asarray(probs, dtype=np.float32)
    V = p.shape[-1]
    if not 1 <= k <= V:
        raise ValueError("need 1 <= k <= V")
    if np.isnan(p).any():
        raise ValueError("NaN in probabilities")
    flat = p.reshape(-1, V)
    ids = np.empty((flat.shape[0], k), dtype=np.int32)
    vals = np.empty((flat.shape[0], k), dtype=np.float32)
    for r in range(flat.shape[0]):
        # stable sort of the negated values keeps equal values in id order
        order = np.argsort(-flat[r], kind="stable")[:k]
        ids[r] = order
        vals[r] = flat[r, order]
    return vals.reshape(p.shape[:-1] + (k,)), ids.reshape(p.shape[:-1] + (k,))
