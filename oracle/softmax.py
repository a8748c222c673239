"""Oracle: processed distributions, p = softmax(logits / T) per row.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Follows "[SGLang] Multi-Layer EAGLE", section 3 (each draft pass runs the
per-step softmax before ``fast_topk``) and zero-to-sglang ch.10, section 5.1
(the acceptance test compares the target's probability of a token with the
draft's, both processed distributions).  The temperature divides the logits
before the softmax, as the configs' "softmax at temperature T" states.

Definition, in float64: p_i = exp((x_i - m) / T) / sum_j exp((x_j - m) / T),
m = max_j x_j.  Subtracting m changes nothing in exact arithmetic and keeps
every exponent <= 0.  Entries at -inf have p = 0; every row needs one finite
entry; NaN is outside the definition.
"""
from __future__ import annotations

import numpy as np


def softmax_rows(logits: np.ndarray, temperature: float = 1.0) -> np.ndarray:
    """softmax(logits / temperature) along the last axis, float64 [..., V]."""
    t = float(temperature)
    if not (np.isfinite(t) and t > 0.0):
        raise ValueError("temperature must be finite and positive")
    x = np.asarray(logits, dtype=np.float32).astype(np.float64)
    if x.shape[-1] < 1:
        raise ValueError("rows need at least one entry")
    if np.isnan(x).any():
        raise ValueError("NaN in logits")
    flat = x.reshape(-1, x.shape[-1])
    out = np.empty(flat.shape, dtype=np.float64)
    for r in range(flat.shape[0]):
        row = flat[r]
        m = row.max()
        if not np.isfinite(m):
            raise ValueError("row %d has no finite entry" % r)
        e = np.exp((row - m) / t)          # exp(-inf) = 0 for masked entries
        out[r] = e / e.sum()
    return out.reshape(x.shape)
