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


def _bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def draft_topk_from_logits(logits: np.ndarray, k: int, temperature: float = 1.0, bf16: bool = False):
    """Fused draft step: softmax(logits / T) of every row and its top-k.

    "[SGLang] Multi-Layer EAGLE", section 3: after each draft pass the logits
    go through the per-step softmax and ``fast_topk``; the temperature is the
    sampling temperature of the draft distribution (the processed rows of the
    workloads are softmax(logits / T)).  This function takes both steps at
    once, without rounding the probabilities in between.

    Definition: with p_i = exp((x_i - max_j x_j) / T) / sum_j exp(...), in
    float64, the k entries that come first when the row is ordered by p
    descending, then id ascending.  For T > 0, p is strictly increasing in x,
    so the order is that of the logits (equal logits: lower id first).

    ``logits``: [..., V] fp32 values, or bf16 bit patterns (uint16) when
    ``bf16``.  Entries may be -inf (excluded vocabulary, p = 0); every row
    needs one finite entry; no NaN.  Returns ``(topk_p [..., k] float64,
    topk_id [..., k] int32)``.
    """
    if not temperature > 0.0:
        raise ValueError("temperature must be positive")
    x = _bf16_bits_to_f64(logits) if bf16 else np.asarray(logits, dtype=np.float32).astype(np.float64)
    V = x.shape[-1]
    if not 1 <= k <= V:
        raise ValueError("need 1 <= k <= V")
    if np.isnan(x).any():
        raise ValueError("NaN in logits")
    flat = x.reshape(-1, V)
    ids = np.empty((flat.shape[0], k), dtype=np.int32)
    vals = np.empty((flat.shape[0], k), dtype=np.float64)
    for r in range(flat.shape[0]):
        row = flat[r]
        m = row.max()
        if not np.isfinite(m):
            raise ValueError("a row has no finite logit")
        e = np.exp((row - m) / float(temperature))        # exp(-inf) = 0
        order = np.argsort(-row, kind="stable")[:k]
        ids[r] = order
        vals[r] = e[order] / e.sum()
    return vals.reshape(x.shape[:-1] + (k,)), ids.reshape(x.shape[:-1] + (k,))
