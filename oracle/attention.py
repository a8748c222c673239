"""Oracle: tree-masked verify attention, dense, in float64.

Follows "EAGLE speculative decoding in four parts": verification is one target
forward over 1 + the candidate count tokens per request ("Exercises",
question 1) with a tree attention mask ("Self-test" answer 1; "Drafting,
verification and slots"), and the pass costs what batch size and tree size
make it ("Design trade-offs").  "[SGLang] Multi-Layer EAGLE", section 6: the
target runs in TARGET_VERIFY mode with the tree's custom mask.

Definition.  Query node i of request b, head h, sees every prefix key
(logical positions 0 .. L_b-1) and the tree keys j with mask[i][j] = 1 (tree
node j's K/V sit at logical position L_b + j).  With scale s,
    out = sum_j softmax_j(s * q.k_j) v_j,   lse = log sum_j exp(s * q.k_j).
Readings: s = 1/sqrt(D); query head h reads KV head h // (Hq/Hkv); a logical
position p of request b lives in pool slot page_table[b][p // P] * P + p % P
of a token-major [slot, Hkv, D] pool.  Inputs are bf16 (upcast exactly);
everything else is float64.
"""
from __future__ import annotations

import numpy as np


def _bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def slot_of(page_table, b: int, pos: np.ndarray, page: int) -> np.ndarray:
    pos = np.asarray(pos, dtype=np.int64)
    return page_table[b, pos // page].astype(np.int64) * page + pos % page


def tree_verify_attention(q, k_pool, v_pool, page_table, prefix_len, mask, page: int = 1,
                          sm_scale=None, requests=None):
    """Dense reference.

    q [B,N,Hq,D], k_pool/v_pool [slots,Hkv,D]: bf16 bit patterns (uint16).
    page_table [B, max_pages] int32; prefix_len [B]; mask [B,N,N] (0/1).
    Returns (out [B,N,Hq,D] f64, lse [B,N,Hq] f64); requests not listed in
    ``requests`` (when given) are left as NaN.
    """
    B, N, Hq, D = q.shape
    Hkv = k_pool.shape[1]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    scale = 1.0 / np.sqrt(D) if sm_scale is None else float(sm_scale)
    out = np.full((B, N, Hq, D), np.nan)
    lse = np.full((B, N, Hq), np.nan)
    for b in (range(B) if requests is None else requests):
        L = int(prefix_len[b])
        slots = slot_of(page_table, b, np.arange(L + N), page)
        K = _bf16_to_f64(k_pool[slots])            # [L+N, Hkv, D]
        Vv = _bf16_to_f64(v_pool[slots])
        Q = _bf16_to_f64(q[b])                     # [N, Hq, D]
        visible = np.concatenate([np.ones((N, L), bool), np.asarray(mask[b]) != 0], axis=1)
        for h in range(Hq):
            kv = h // G
            s = scale * (Q[:, h, :] @ K[:, kv, :].T)          # [N, L+N]
            s = np.where(visible, s, -np.inf)
            m = s.max(axis=1, keepdims=True)
            e = np.exp(s - m)
            z = e.sum(axis=1, keepdims=True)
            out[b, :, h, :] = (e / z) @ Vv[:, kv, :]
            lse[b, :, h] = (m + np.log(z))[:, 0]
    return out, lse
