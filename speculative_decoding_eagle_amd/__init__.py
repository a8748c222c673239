"""EAGLE-style draft-tree build and target-side verify on MI355X (gfx950).

The compute lives in libsdv.so (HIP kernels behind the C ABI of
include/sdv.h); this package holds the kernels' sources (``csrc/``), the
in-tree build (``build``) and a thin torch binding (``binding``) whose
functions carry the C entry points' names.  Importing the package does not
open the library; the first binding call does, and fails loudly if it has
not been built.
"""
from .binding import (  # noqa: F401
    GREEDY,
    KVAlloc,
    STOCHASTIC,
    SdvError,
    STATUS_ACCEPT_WAIT,
    STATUS_ATTN_MERGE_WAIT,
    STATUS_TLI_REUSE,
    STATUS_TOPK_MERGE_WAIT,
    device_status,
    sdv_set_wait_limit,
    sdv_tli_check,
    sdv_workspace_status,
    sdv_build_chain,
    sdv_build_tree,
    sdv_compact_kv,
    sdv_draft_extend_prep,
    sdv_draft_topk,
    sdv_draft_topk_logits,
    sdv_softmax_rows,
    sdv_kv_alloc_backup,
    sdv_kv_alloc_branches,
    sdv_kv_alloc_extend,
    sdv_kv_alloc_free,
    sdv_kv_alloc_init,
    sdv_kv_alloc_restore,
    sdv_kv_branch_pages,
    sdv_tli_build_maps,
    sdv_tli_constrain_draft_logits,
    sdv_tli_lm_head,
    sdv_tli_map_ids,
    sdv_tli_q_scatter,
    sdv_tree_verify_attention,
    sdv_verify_accept,
    sdv_verify_accept_noalloc,
)
