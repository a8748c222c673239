"""Oracle: Token-Level Intersection (TLI) for heterogeneous vocabularies.

Follows sglang PR #22883 "TLI (Token-Level Intersection)", "Modifications":
* the vocabulary mapping exposes ``constrain_draft_logits`` (logits outside the
  intersection become -inf), ``map_target_to_draft_ids``,
  ``map_draft_to_target_ids`` and the sorted ``intersection_draft_ids`` (the
  columns kept by the pruned LM head); models without an unknown token fall
  back to the EOS id;
* the draft LM head is replaced by a compact [intersection_size x hidden_dim]
  matrix, turning the draft's dominant matmul from O(B * V_draft * H) into
  O(B * K * H);
* the target's rejection-sampling step is unchanged, which keeps TLI lossless
  ("Motivation"; "Accuracy Tests").

Readings where the pages leave a step open: the intersection is given as pairs
(inter_ids[j], tgt_ids[j]) -- draft id and target id of the same normalised
token -- with inter_ids sorted; the pruned weight is row-major [K, H] with row
j belonging to draft id inter_ids[j]; a draft id outside the intersection maps
to target id -1 and a target id outside it maps to the caller's fallback draft
id; the draft distribution over the K intersection ids is carried into the
target vocabulary (zero elsewhere) so the verify step runs unchanged.
"""
from __future__ import annotations

import numpy as np


def _bf16_to_f64(bits):
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def build_maps(inter_ids, tgt_ids, V_draft: int, V_target: int, fallback: int):
    """d2t [V_draft] (-1 outside the intersection), t2d [V_target] (fallback outside)."""
    d2t = np.full(V_draft, -1, np.int32)
    t2d = np.full(V_target, int(fallback), np.int32)
    for d, t in zip(np.asarray(inter_ids).tolist(), np.asarray(tgt_ids).tolist()):
        d2t[d] = t
        t2d[t] = d
    return d2t, t2d


def check_tli_shape(topk: int, num_steps: int, num_draft_tokens: int) -> None:
    """The TLI validation rules (sglang PR #22883, "Modified files", the
    validation block added to the server-argument checks): TLI drafts a single
    candidate per step (topk must be 1) and the draft is a chain with the root,
    so num_draft_tokens must equal num_steps + 1.  Raises ValueError otherwise."""
    if int(topk) != 1:
        raise ValueError("TLI needs topk == 1 (got %d)" % topk)
    if int(num_steps) < 1 or int(num_draft_tokens) != int(num_steps) + 1:
        raise ValueError("TLI needs num_draft_tokens == num_steps + 1 (got %d, %d)"
                         % (num_draft_tokens, num_steps))


def map_ids(table, ids):
    """out[i] = table[ids[i]]; an id outside [0, len(table)) maps to -1.

    Reading: an id that names no entry of the table (the -1 padding of the
    accept walk's committed-token array, or any other value out of range) has
    no image in the other vocabulary and stays the padding value -1, so id
    arrays can be remapped whole, padding included."""
    ids = np.asarray(ids, np.int64)
    table = np.asarray(table, np.int32)
    out = np.full(ids.shape, -1, np.int32)
    ok = (ids >= 0) & (ids < len(table))
    out[ok] = table[ids[ok]]
    return out


def constrain_logits(pruned, inter_ids, V_draft: int):
    """Dense draft logits [B, V_draft]: pruned[b, j] at inter_ids[j], -inf elsewhere."""
    pruned = np.asarray(pruned, np.float32)
    out = np.full((pruned.shape[0], V_draft), -np.inf, np.float32)
    out[:, np.asarray(inter_ids, np.int64)] = pruned
    return out


def q_scatter(q_pruned, tgt_ids, V_target: int):
    """Target-vocab rows [rows, V_target]: q_pruned[r, j] at tgt_ids[j], 0 elsewhere."""
    q_pruned = np.asarray(q_pruned, np.float32)
    out = np.zeros((q_pruned.shape[0], V_target), np.float32)
    out[:, np.asarray(tgt_ids, np.int64)] = q_pruned
    return out


def lm_head(hidden_bits, weight_bits):
    """Pruned LM head in float64: logits[b, j] = sum_h hidden[b, h] * W[j, h]."""
    return _bf16_to_f64(hidden_bits) @ _bf16_to_f64(weight_bits).T
