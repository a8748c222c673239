"""ctypes loader of libsdv.so and the C declarations of its entry points.

torch is imported before the library is opened: the HIP runtime torch
loaded is then the one libsdv.so binds to (both carry the soname
libamdhip64.so.7), so device pointers and streams are shared.
"""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (must precede the CDLL below)

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsdv.so")

c_i32, c_i64, c_sz, c_p, c_f32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_float


class TreeShape(ctypes.Structure):
    _fields_ = [("B", c_i32), ("k", c_i32), ("S", c_i32), ("N", c_i32)]


class AttnShape(ctypes.Structure):
    _fields_ = [("B", c_i32), ("N", c_i32), ("Hq", c_i32), ("Hkv", c_i32), ("D", c_i32), ("page", c_i32),
                ("max_pages", c_i32), ("num_slots", c_i64)]


class AcceptShape(ctypes.Structure):
    _fields_ = [("B", c_i32), ("N", c_i32), ("S", c_i32), ("V", c_i32), ("R", c_i32), ("mode", c_i32)]


class KVShape(ctypes.Structure):
    _fields_ = [("B", c_i32), ("N", c_i32), ("S", c_i32), ("page", c_i32), ("Hkv", c_i32), ("D", c_i32),
                ("layers", c_i32), ("max_pages", c_i32), ("num_slots", c_i64)]


class BranchShape(ctypes.Structure):
    _fields_ = [("B", c_i32), ("page", c_i32), ("topk", c_i32), ("S", c_i32), ("Hkv", c_i32), ("D", c_i32),
                ("layers", c_i32), ("max_pages", c_i32), ("num_slots", c_i64)]


# name -> (restype, argtypes)
SIGNATURES = {
    "sdv_last_error": (ctypes.c_char_p, []),
    "sdv_version": (c_i32, []),
    "sdv_workspace_status": (c_i32, [c_p, c_sz, ctypes.POINTER(ctypes.c_uint32), c_i32, c_p]),
    "sdv_set_wait_limit": (ctypes.c_uint32, [ctypes.c_uint32]),
    "sdv_tli_check": (c_i32, [c_i32, c_i32, c_i32]),
    "sdv_draft_topk_workspace_size": (c_sz, [c_i64, c_i32, c_i32]),
    "sdv_draft_topk": (c_i32, [c_p, c_i64, c_i32, c_i32, c_p, c_p, c_p, c_sz, c_p]),
    "sdv_draft_topk_logits_workspace_size": (c_sz, [c_i64, c_i32, c_i32]),
    "sdv_draft_topk_logits": (c_i32, [c_p, c_i32, c_i64, c_i32, c_i32, c_f32, c_p, c_p, c_p, c_sz, c_p]),
    "sdv_softmax_rows": (c_i32, [c_p, c_i64, c_i32, c_f32, c_p, c_p]),
    "sdv_build_tree": (c_i32, [TreeShape] + [c_p] * 15 + [c_p]),
    "sdv_tree_verify_attention_workspace_size": (c_sz, [AttnShape]),
    "sdv_tree_verify_attention": (c_i32, [AttnShape, c_f32] + [c_p] * 8 + [c_p, c_sz, c_p]),
    "sdv_verify_accept_workspace_size": (c_sz, [AcceptShape]),
    "sdv_verify_accept": (c_i32, [AcceptShape, c_i32] + [c_p] * 14 + [c_p, c_sz, c_p]),
    "sdv_verify_accept_noalloc": (c_i32, [AcceptShape, c_i32] + [c_p] * 14 + [c_p]),
    "sdv_compact_kv_workspace_size": (c_sz, [KVShape]),
    "sdv_compact_kv": (c_i32, [KVShape] + [c_p] * 9 + [c_p, c_sz, c_p]),
    "sdv_tli_lm_head": (c_i32, [c_i32, c_i32, c_i32, c_p, c_p, c_p, c_p]),
    "sdv_tli_build_maps": (c_i32, [c_i32, c_p, c_p, c_i32, c_i32, c_i32, c_p, c_p, c_p]),
    "sdv_tli_map_ids": (c_i32, [c_p, c_i32, c_p, c_i64, c_p, c_p]),
    "sdv_build_chain": (c_i32, [c_i32, c_i32] + [c_p] * 15 + [c_p]),
    "sdv_kv_branch_pages": (c_i32, [c_i32, c_i32]),
    "sdv_kv_alloc_init": (c_i32, [c_i32, c_p, c_p, c_p]),
    "sdv_kv_alloc_backup": (c_i32, [c_p, c_p, c_p]),
    "sdv_kv_alloc_restore": (c_i32, [c_i32, c_p, c_p, c_p]),
    "sdv_kv_alloc_free": (c_i32, [c_i32, c_p, c_p, c_p, c_p, c_i32, c_p]),
    "sdv_kv_alloc_extend": (c_i32, [c_i32, c_p, c_p, c_i32, c_i32, c_i32, c_p, c_i32, c_p, c_p, c_p]),
    "sdv_kv_alloc_branches": (c_i32, [c_i32, c_p, c_p, BranchShape] + [c_p] * 7),
    "sdv_draft_extend_prep": (c_i32, [c_i32, c_i32, c_i32] + [c_p] * 5 + [c_i32] + [c_p] * 7),
    "sdv_tli_constrain_draft_logits": (c_i32, [c_i32, c_i32, c_i32, c_p, c_p, c_p, c_p]),
    "sdv_tli_q_scatter_workspace_size": (c_sz, [c_i32]),
    "sdv_tli_q_scatter": (c_i32, [c_i64, c_i32, c_i32, c_p, c_p, c_p, c_p, c_sz, c_p]),
}

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libsdv.so is not built (run `python -m speculative_decoding_eagle_amd.build`)")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib
