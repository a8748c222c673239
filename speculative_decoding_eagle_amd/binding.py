"""Thin torch-tensor binding of the C ABI in include/sdv.h.

Each function has the name of the C entry point it calls and only marshals
arguments: it checks dtypes, devices and contiguity, allocates outputs and
workspaces that the caller did not pass (torch device memory), and passes raw
pointers plus the current HIP stream.  All computation happens in the HIP
kernels; a non-zero status raises ``SdvError`` with the library's message.
bf16 tensors may be given as torch.bfloat16 or as int16/uint16 bit patterns.
"""
from __future__ import annotations

import ctypes
import math
from typing import Optional, Sequence

import torch

from . import _lib
from ._lib import AcceptShape, AttnShape, KVShape, TreeShape

GREEDY, STOCHASTIC = 0, 1


class SdvError(RuntimeError):
    pass


def _check(rc: int, what: str):
    if rc != 0:
        msg = _lib.lib().sdv_last_error().decode(errors="replace")
        raise SdvError("%s failed (status %d): %s" % (what, rc, msg))


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _ptr(t: Optional[torch.Tensor], dtype=None, name="tensor", allow_none=False) -> int:
    if t is None:
        if allow_none:
            return 0
        raise ValueError("%s is required" % name)
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None:
        ok = t.dtype in dtype if isinstance(dtype, tuple) else t.dtype == dtype
        if not ok:
            raise ValueError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))
    return t.data_ptr()


BF16 = (torch.bfloat16, torch.int16, torch.uint16)


def _workspace(nbytes: int, device, ws: Optional[torch.Tensor]):
    if nbytes == 0:
        return 0, 0
    if ws is None:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    if ws.numel() * ws.element_size() < nbytes:
        raise ValueError("workspace too small: %d bytes needed" % nbytes)
    return ws.data_ptr(), ws.numel() * ws.element_size()


def _keep(*_):
    """Holds references until the call returns (workspaces live on the stream)."""


# ------------------------------------------------------- status and checks

STATUS_ACCEPT_WAIT, STATUS_ATTN_MERGE_WAIT, STATUS_TOPK_MERGE_WAIT, STATUS_TLI_REUSE = 1, 2, 4, 8


def _ws_status(ws: torch.Tensor, stream: int, reset: bool) -> int:
    st = ctypes.c_uint32(0)
    nbytes = ws.numel() * ws.element_size()
    _check(_lib.lib().sdv_workspace_status(_ptr(ws, name="ws"), nbytes, ctypes.byref(st), int(bool(reset)),
                                           stream), "sdv_workspace_status")
    return int(st.value)


def sdv_workspace_status(ws: torch.Tensor, reset: bool = True) -> int:
    """Status bits of a workspace (synchronises its device's current stream);
    with ``reset`` a non-zero status zero-fills the workspace again."""
    return _ws_status(ws, _stream(ws.device), reset)


def device_status(device=None, reset: bool = True) -> int:
    """OR of the status words of the workspaces this binding keeps for
    ``device`` (on the stream each belongs to); reset as in
    ``sdv_workspace_status``."""
    dev = torch.device(device if device is not None else "cuda")
    idx = dev.index if dev.index is not None else torch.cuda.current_device()
    bits = 0
    for cache in (_TOPK_WS, _ATTN_WS, _ACC_WS):
        for (d, stream), ws in list(cache.items()):
            if d == idx:
                bits |= _ws_status(ws, stream, reset)
    return bits


def sdv_set_wait_limit(polls: int) -> int:
    """Process-wide poll limit of the bounded waits (0xFFFFFFFF: library
    default; 0: give up at once).  Returns the previous setting."""
    return int(_lib.lib().sdv_set_wait_limit(int(polls) & 0xFFFFFFFF))


def sdv_tli_check(topk: int, num_steps: int, num_draft_tokens: int) -> None:
    """Raises SdvError unless topk == 1 and num_draft_tokens == num_steps + 1."""
    _check(_lib.lib().sdv_tli_check(int(topk), int(num_steps), int(num_draft_tokens)), "sdv_tli_check")


# ---------------------------------------------------------------------- A1

_TOPK_WS = {}


def sdv_draft_topk(probs: torch.Tensor, k: int, topk_p=None, topk_id=None, ws=None):
    """Top-k of every row of ``probs`` [..., V] fp32 -> (topk_p, topk_id) [..., k].

    ``ws``: a zero-filled workspace of the size query's bytes (the calls keep
    it zero-filled); by default a cached one per (device, stream)."""
    V = probs.shape[-1]
    rows = probs.numel() // V if V else 0
    dev = probs.device
    if topk_p is None:
        topk_p = torch.empty(probs.shape[:-1] + (k,), dtype=torch.float32, device=dev)
    if topk_id is None:
        topk_id = torch.empty(probs.shape[:-1] + (k,), dtype=torch.int32, device=dev)
    L = _lib.lib()
    need = L.sdv_draft_topk_workspace_size(rows, V, k)
    if need and ws is None:
        ws = _zeroed_workspace(_TOPK_WS, need, dev)
    wp, wb = _workspace(need, dev, ws)
    _check(L.sdv_draft_topk(_ptr(probs, torch.float32, "probs"), rows, V, k, _ptr(topk_p, torch.float32, "topk_p"),
                            _ptr(topk_id, torch.int32, "topk_id"), wp, wb, _stream(dev)), "sdv_draft_topk")
    return topk_p, topk_id


def sdv_draft_topk_logits(logits: torch.Tensor, k: int, temperature: float = 1.0, topk_p=None, topk_id=None,
                          ws=None):
    """softmax(logits / temperature) top-k of every row of ``logits`` [..., V]
    (fp32 or bf16) -> (topk_p fp32, topk_id int32) [..., k]."""
    V = logits.shape[-1]
    rows = logits.numel() // V if V else 0
    dev = logits.device
    if logits.dtype == torch.float32:
        dtype = 0
    elif logits.dtype == torch.bfloat16:
        dtype = 1
    else:
        raise ValueError("logits must be float32 or bfloat16, got %s" % logits.dtype)
    if topk_p is None:
        topk_p = torch.empty(logits.shape[:-1] + (k,), dtype=torch.float32, device=dev)
    if topk_id is None:
        topk_id = torch.empty(logits.shape[:-1] + (k,), dtype=torch.int32, device=dev)
    L = _lib.lib()
    need = L.sdv_draft_topk_logits_workspace_size(rows, V, k)
    if need and ws is None:
        ws = _zeroed_workspace(_TOPK_WS, need, dev)
    wp, wb = _workspace(need, dev, ws)
    _check(L.sdv_draft_topk_logits(_ptr(logits, (torch.float32, torch.bfloat16), "logits"), dtype, rows, V, k,
                                   float(temperature), _ptr(topk_p, torch.float32, "topk_p"),
                                   _ptr(topk_id, torch.int32, "topk_id"), wp, wb, _stream(dev)),
           "sdv_draft_topk_logits")
    return topk_p, topk_id


def sdv_softmax_rows(logits: torch.Tensor, temperature: float = 1.0, out=None):
    """softmax(logits / temperature) of every row of ``logits`` [..., V] (fp32)
    -> fp32 tensor of the same shape."""
    V = logits.shape[-1]
    rows = logits.numel() // V if V else 0
    dev = logits.device
    if out is None:
        out = torch.empty(logits.shape, dtype=torch.float32, device=dev)
    if out.shape != logits.shape:
        raise ValueError("out must have the shape of logits")
    L = _lib.lib()
    _check(L.sdv_softmax_rows(_ptr(logits, torch.float32, "logits"), rows, V, float(temperature),
                              _ptr(out, torch.float32, "out"), _stream(dev)), "sdv_softmax_rows")
    return out


# -------------------------------------------------------------------- A2-A4

TREE_OUTPUTS = ("tokens", "parent", "depth", "positions", "score", "q_row", "mask", "mask_bits",
                "retrieve_index", "next_token", "next_sibling")


def _tree_outputs(B: int, N: int, dev, out, with_mask: bool):
    out = dict(out or {})
    W = (N + 31) // 32
    i32 = torch.int32
    shapes = {"tokens": ((B, N), i32), "parent": ((B, N), i32), "depth": ((B, N), i32),
              "positions": ((B, N), i32), "score": ((B, N), torch.float32), "q_row": ((B, N), i32),
              "mask_bits": ((B, N, W), i32), "retrieve_index": ((B, N), i32), "next_token": ((B, N), i32),
              "next_sibling": ((B, N), i32)}
    if with_mask:
        shapes["mask"] = ((B, N, N), torch.uint8)
    for name, (shape, dtype) in shapes.items():
        if name not in out:
            out[name] = torch.empty(shape, dtype=dtype, device=dev)
    return out


def _tree_output_ptrs(out):
    return [_ptr(out[n]) for n in ("tokens", "parent", "depth", "positions", "score", "q_row")] + [
        _ptr(out.get("mask"), torch.uint8, "mask", allow_none=True),
        _ptr(out["mask_bits"], (torch.int32, torch.uint32), "mask_bits"),
        _ptr(out["retrieve_index"]), _ptr(out["next_token"]), _ptr(out["next_sibling"])]


def sdv_build_tree(topk_p, topk_id, root_token, prefix_len, k: int, S: int, N: int, out=None,
                   with_mask: bool = True):
    """Candidate tree and verify arrays; returns a dict of device tensors."""
    B = topk_p.shape[0]
    out = _tree_outputs(B, N, topk_p.device, out, with_mask)
    i32 = torch.int32
    _check(_lib.lib().sdv_build_tree(
        TreeShape(B, k, S, N), _ptr(topk_p, torch.float32, "topk_p"), _ptr(topk_id, i32, "topk_id"),
        _ptr(root_token, i32, "root_token"), _ptr(prefix_len, i32, "prefix_len"), *_tree_output_ptrs(out),
        _stream(topk_p.device)), "sdv_build_tree")
    return out


def sdv_build_chain(topk_p, topk_id, root_token, prefix_len, out=None, with_mask: bool = True):
    """Multi-layer draft chain from each step's top-1 ([B, S] or [B, S, 1]);
    returns the same dict as sdv_build_tree with N = S + 1."""
    B, S = topk_p.shape[0], topk_p.shape[1]
    if topk_p.dim() == 3 and topk_p.shape[2] != 1:
        raise ValueError("a chain takes one token per step")
    out = _tree_outputs(B, S + 1, topk_p.device, out, with_mask)
    i32 = torch.int32
    _check(_lib.lib().sdv_build_chain(
        B, S, _ptr(topk_p, torch.float32, "topk_p"), _ptr(topk_id, i32, "topk_id"),
        _ptr(root_token, i32, "root_token"), _ptr(prefix_len, i32, "prefix_len"), *_tree_output_ptrs(out),
        _stream(topk_p.device)), "sdv_build_chain")
    return out


# ---------------------------------------------------------------------- A5

_ATTN_WS = {}
_ACC_WS = {}


def _zeroed_workspace(cache, nbytes: int, device) -> torch.Tensor:
    """A zero-filled workspace kept per (device, stream) for entry points whose
    calls leave it zero-filled: cleared once, when (re)allocated."""
    key = (device.index, torch.cuda.current_stream(device).cuda_stream)
    ws = cache.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(max(nbytes, 1 << 16), dtype=torch.uint8, device=device)
        cache[key] = ws
    return ws


def _attn_workspace(nbytes: int, device) -> torch.Tensor:
    """Zero-filled attention workspace, one per (device, stream): every call
    leaves it zero-filled again, so it is cleared once, when allocated."""
    return _zeroed_workspace(_ATTN_WS, nbytes, device)


def sdv_tree_verify_attention(q, k_pool, v_pool, page_table, prefix_len, mask_bits, page: int = 1,
                              sm_scale: float = 0.0, out=None, lse=None, want_lse: bool = False, ws=None,
                              split_keys: bool = True):
    """Tree-masked attention; returns (out [B,N,Hq,D] bf16, lse or None).

    ``ws``: a zero-filled workspace of the size query's bytes (kept
    zero-filled by the calls); by default a cached one.  ``split_keys=False``
    passes no workspace, which runs without the key split."""
    B, N, Hq, D = q.shape
    Hkv = k_pool.shape[1]
    dev = q.device
    if out is None:
        out = torch.empty((B, N, Hq, D), dtype=torch.bfloat16, device=dev)
    if lse is None and want_lse:
        lse = torch.empty((B, N, Hq), dtype=torch.float32, device=dev)
    shape = AttnShape(B, N, Hq, Hkv, D, page, page_table.shape[1], k_pool.shape[0])
    L = _lib.lib()
    need = L.sdv_tree_verify_attention_workspace_size(shape)
    if not split_keys or need == 0:
        wp, wb = 0, 0
    else:
        if ws is None:
            ws = _attn_workspace(need, dev)
        wp, wb = _workspace(need, dev, ws)
    _check(L.sdv_tree_verify_attention(
        shape, float(sm_scale), _ptr(q, BF16, "q"), _ptr(k_pool, BF16, "k_pool"), _ptr(v_pool, BF16, "v_pool"),
        _ptr(page_table, torch.int32, "page_table"), _ptr(prefix_len, torch.int32, "prefix_len"),
        _ptr(mask_bits, (torch.int32, torch.uint32), "mask_bits"), _ptr(out, BF16, "out"),
        _ptr(lse, torch.float32, "lse", allow_none=True), wp, wb, _stream(dev)), "sdv_tree_verify_attention")
    _keep(ws)
    return out, lse


# -------------------------------------------------------------------- A6-A7

def sdv_verify_accept(mode: int, tree, target, S: int, eos_id: int = -1, remaining=None, draft_probs=None,
                      u_accept=None, u_draw=None, out=None, ws=None):
    """Accept walk; ``tree`` holds tokens/next_token/next_sibling/q_row [B,N].
    Returns dict accept_len, accept_path, commit_tokens, commit_len, next_root."""
    tokens = tree["tokens"]
    B, N = tokens.shape
    V = target.shape[-1]
    R = draft_probs.shape[1] if draft_probs is not None else 0
    dev = tokens.device
    out = dict(out or {})
    i32 = torch.int32
    for name, shape in (("accept_len", (B,)), ("accept_path", (B, S + 1)), ("commit_tokens", (B, S + 1)),
                        ("commit_len", (B,)), ("next_root", (B,))):
        if name not in out:
            out[name] = torch.empty(shape, dtype=i32, device=dev)
    shape = AcceptShape(B, N, S, V, R, mode)
    L = _lib.lib()
    need = L.sdv_verify_accept_workspace_size(shape)
    if ws is None and need:
        ws = _zeroed_workspace(_ACC_WS, need, dev)
    wp, wb = _workspace(need, dev, ws)
    _check(L.sdv_verify_accept(
        shape, eos_id, _ptr(remaining, i32, "remaining", allow_none=True), _ptr(tokens, i32, "tokens"),
        _ptr(tree["next_token"], i32, "next_token"), _ptr(tree["next_sibling"], i32, "next_sibling"),
        _ptr(tree.get("q_row"), i32, "q_row", allow_none=True), _ptr(target, torch.float32, "target"),
        _ptr(draft_probs, torch.float32, "draft_probs", allow_none=True),
        _ptr(u_accept, torch.float32, "u_accept", allow_none=True),
        _ptr(u_draw, torch.float32, "u_draw", allow_none=True),
        _ptr(out["accept_len"]), _ptr(out["accept_path"]), _ptr(out["commit_tokens"]), _ptr(out["commit_len"]),
        _ptr(out["next_root"]), wp, wb, _stream(dev)), "sdv_verify_accept")
    return out


def sdv_verify_accept_noalloc(mode: int, tree, target, S: int, eos_id: int = -1, remaining=None,
                              draft_probs=None, u_accept=None, u_draw=None, out=None):
    """The accept walk without a workspace (the library's static scratch, at
    most 1024 requests).  Outputs must be passed in ``out`` (this entry point
    is for callers that allocate nothing); returns ``out``."""
    tokens = tree["tokens"]
    B, N = tokens.shape
    V = target.shape[-1]
    R = draft_probs.shape[1] if draft_probs is not None else 0
    i32 = torch.int32
    shape = AcceptShape(B, N, S, V, R, mode)
    _check(_lib.lib().sdv_verify_accept_noalloc(
        shape, eos_id, _ptr(remaining, i32, "remaining", allow_none=True), _ptr(tokens, i32, "tokens"),
        _ptr(tree["next_token"], i32, "next_token"), _ptr(tree["next_sibling"], i32, "next_sibling"),
        _ptr(tree.get("q_row"), i32, "q_row", allow_none=True), _ptr(target, torch.float32, "target"),
        _ptr(draft_probs, torch.float32, "draft_probs", allow_none=True),
        _ptr(u_accept, torch.float32, "u_accept", allow_none=True),
        _ptr(u_draw, torch.float32, "u_draw", allow_none=True),
        _ptr(out["accept_len"], i32, "accept_len"), _ptr(out["accept_path"], i32, "accept_path"),
        _ptr(out["commit_tokens"], i32, "commit_tokens"), _ptr(out["commit_len"], i32, "commit_len"),
        _ptr(out["next_root"], i32, "next_root"), _stream(tokens.device)), "sdv_verify_accept_noalloc")
    return out


# ------------------------------------------------------- KV allocation

class KVAlloc:
    """Device allocator state: free_ids [capacity] and state [4] int32
    ({top, pushes, error, 0}); see sdv_kv_alloc_* in include/sdv.h."""

    def __init__(self, capacity: int, device="cuda"):
        self.capacity = capacity
        self.free_ids = torch.empty(max(1, capacity), dtype=torch.int32, device=device)
        self.state = torch.empty(4, dtype=torch.int32, device=device)

    def ptrs(self):
        return self.capacity, _ptr(self.free_ids, torch.int32, "free_ids"), _ptr(self.state, torch.int32, "state")


def sdv_kv_alloc_init(capacity: int, device="cuda") -> KVAlloc:
    a = KVAlloc(capacity, device)
    _check(_lib.lib().sdv_kv_alloc_init(*a.ptrs(), _stream(a.state.device)), "sdv_kv_alloc_init")
    return a


def sdv_kv_alloc_backup(a: KVAlloc, backup=None):
    if backup is None:
        backup = torch.empty(2, dtype=torch.int32, device=a.state.device)
    _check(_lib.lib().sdv_kv_alloc_backup(_ptr(a.state, torch.int32, "state"), _ptr(backup, torch.int32, "backup"),
                                          _stream(a.state.device)), "sdv_kv_alloc_backup")
    return backup


def sdv_kv_alloc_restore(a: KVAlloc, backup):
    _check(_lib.lib().sdv_kv_alloc_restore(a.capacity, _ptr(a.state, torch.int32, "state"),
                                           _ptr(backup, torch.int32, "backup"), _stream(a.state.device)),
           "sdv_kv_alloc_restore")


def sdv_kv_alloc_free(a: KVAlloc, ids, num_ids):
    """Releases ids[0 .. num_ids[0]) (num_ids a device int32 tensor)."""
    _check(_lib.lib().sdv_kv_alloc_free(*a.ptrs(), _ptr(ids, torch.int32, "ids"), _ptr(num_ids, torch.int32, "num_ids"),
                                        ids.numel(), _stream(a.state.device)), "sdv_kv_alloc_free")


def sdv_kv_alloc_extend(a: KVAlloc, page: int, n: int, page_table, seq_len, out_loc=None):
    B, max_pages = page_table.shape
    if out_loc is None:
        out_loc = torch.empty((B, n), dtype=torch.int32, device=page_table.device)
    _check(_lib.lib().sdv_kv_alloc_extend(*a.ptrs(), B, page, n, _ptr(page_table, torch.int32, "page_table"),
                                          max_pages, _ptr(seq_len, torch.int32, "seq_len"),
                                          _ptr(out_loc, torch.int32, "out_loc"), _stream(page_table.device)),
           "sdv_kv_alloc_extend")
    return out_loc


def sdv_kv_branch_pages(page: int, S: int) -> int:
    return int(_lib.lib().sdv_kv_branch_pages(page, S))


def sdv_kv_alloc_branches(a: KVAlloc, page: int, topk: int, S: int, page_table, seq_len,
                          k_pools: Sequence[torch.Tensor] = (), v_pools: Sequence[torch.Tensor] = (),
                          branch_pages=None, out_loc=None):
    """Per-branch draft regions (and the partial-page copies into the pools).
    Returns (branch_pages [B, topk, maxpb], out_loc [B, topk, S])."""
    B, max_pages = page_table.shape
    dev = page_table.device
    maxpb = sdv_kv_branch_pages(page, S)
    if branch_pages is None:
        branch_pages = torch.empty((B, topk, maxpb), dtype=torch.int32, device=dev)
    if out_loc is None:
        out_loc = torch.empty((B, topk, S), dtype=torch.int32, device=dev)
    layers = len(k_pools)
    if len(v_pools) != layers:
        raise ValueError("K and V pools must match")
    Hkv = k_pools[0].shape[1] if layers else 0
    D = k_pools[0].shape[2] if layers else 0
    slots = k_pools[0].shape[0] if layers else 0
    kp = (ctypes.c_void_p * max(1, layers))(*[_ptr(t, BF16, "k_pool") for t in k_pools])
    vp = (ctypes.c_void_p * max(1, layers))(*[_ptr(t, BF16, "v_pool") for t in v_pools])
    shape = _lib.BranchShape(B, page, topk, S, Hkv, D, layers, max_pages, slots)
    _check(_lib.lib().sdv_kv_alloc_branches(
        *a.ptrs(), shape, ctypes.cast(kp, ctypes.c_void_p), ctypes.cast(vp, ctypes.c_void_p),
        _ptr(page_table, torch.int32, "page_table"), _ptr(seq_len, torch.int32, "seq_len"),
        _ptr(branch_pages, torch.int32, "branch_pages"), _ptr(out_loc, torch.int32, "out_loc"), _stream(dev)),
        "sdv_kv_alloc_branches")
    return branch_pages, out_loc


# ------------------------------------------------- draft extend index prep

EXTEND_OUTPUTS = ("extend_start", "input_ids", "positions", "hidden_index", "last_index", "seq_len")


def sdv_draft_extend_prep(prefix_len, commit_len, commit_tokens, accept_path, N: int, t2d=None, out=None):
    """Packed rows of the draft extend after a verify step.  Returns a dict of
    EXTEND_OUTPUTS; input_ids / positions / hidden_index hold B * (S+1) rows
    of which extend_start[B] are written."""
    B, S1 = commit_tokens.shape
    dev = commit_tokens.device
    out = {} if out is None else out
    sizes = {"extend_start": B + 1, "input_ids": B * S1, "positions": B * S1, "hidden_index": B * S1,
             "last_index": B, "seq_len": B}
    for name in EXTEND_OUTPUTS:
        if out.get(name) is None:
            out[name] = torch.empty(sizes[name], dtype=torch.int32, device=dev)
    vt = 0 if t2d is None else t2d.numel()
    _check(_lib.lib().sdv_draft_extend_prep(
        B, N, S1 - 1, _ptr(prefix_len, torch.int32, "prefix_len"), _ptr(commit_len, torch.int32, "commit_len"),
        _ptr(commit_tokens, torch.int32, "commit_tokens"), _ptr(accept_path, torch.int32, "accept_path"),
        _ptr(t2d, torch.int32, "t2d", allow_none=True), vt,
        *[_ptr(out[name], torch.int32, name) for name in EXTEND_OUTPUTS], _stream(dev)),
        "sdv_draft_extend_prep")
    return out


# ---------------------------------------------------------------------- A8

def sdv_compact_kv(page_table, prefix_len, accept_len, accept_path, N: int, S: int, page: int,
                   k_pools: Sequence[torch.Tensor] = (), v_pools: Sequence[torch.Tensor] = (),
                   new_len=None, freed=None, num_freed=None, ws=None):
    """Compaction in place (page_table and, for page > 1, the pools).
    Returns (new_len [B], freed [B*N], num_freed [1])."""
    B, max_pages = page_table.shape
    dev = page_table.device
    i32 = torch.int32
    if new_len is None:
        new_len = torch.empty(B, dtype=i32, device=dev)
    if freed is None:
        freed = torch.empty(max(1, B * N), dtype=i32, device=dev)
    if num_freed is None:
        num_freed = torch.empty(1, dtype=i32, device=dev)
    layers = len(k_pools)
    if page > 1 and (layers == 0 or len(v_pools) != layers):
        raise ValueError("page > 1 needs matching K and V pools")
    Hkv = k_pools[0].shape[1] if layers else 0
    D = k_pools[0].shape[2] if layers else 0
    slots = k_pools[0].shape[0] if layers else 0
    kp = (ctypes.c_void_p * max(1, layers))(*[_ptr(t, BF16, "k_pool") for t in k_pools])
    vp = (ctypes.c_void_p * max(1, layers))(*[_ptr(t, BF16, "v_pool") for t in v_pools])
    shape = KVShape(B, N, S, page, Hkv, D, layers, max_pages, slots)
    L = _lib.lib()
    wp, wb = _workspace(L.sdv_compact_kv_workspace_size(shape), dev, ws)
    _check(L.sdv_compact_kv(
        shape, ctypes.cast(kp, ctypes.c_void_p), ctypes.cast(vp, ctypes.c_void_p),
        _ptr(page_table, i32, "page_table"), _ptr(prefix_len, i32, "prefix_len"),
        _ptr(accept_len, i32, "accept_len"), _ptr(accept_path, i32, "accept_path"), _ptr(new_len, i32, "new_len"),
        _ptr(freed, i32, "freed"), _ptr(num_freed, i32, "num_freed"), wp, wb, _stream(dev)), "sdv_compact_kv")
    return new_len, freed, num_freed


# ------------------------------------------------------------------- A9-A10

def sdv_tli_lm_head(hidden, weight, logits=None):
    B, H = hidden.shape
    K = weight.shape[0]
    if logits is None:
        logits = torch.empty((B, K), dtype=torch.float32, device=hidden.device)
    _check(_lib.lib().sdv_tli_lm_head(B, H, K, _ptr(hidden, BF16, "hidden"), _ptr(weight, BF16, "weight"),
                                      _ptr(logits, torch.float32, "logits"), _stream(hidden.device)),
           "sdv_tli_lm_head")
    return logits


def sdv_tli_build_maps(inter_ids, tgt_ids, V_draft: int, V_target: int, fallback: int, d2t=None, t2d=None):
    dev = inter_ids.device
    if d2t is None:
        d2t = torch.empty(V_draft, dtype=torch.int32, device=dev)
    if t2d is None:
        t2d = torch.empty(V_target, dtype=torch.int32, device=dev)
    _check(_lib.lib().sdv_tli_build_maps(inter_ids.numel(), _ptr(inter_ids, torch.int32, "inter_ids"),
                                         _ptr(tgt_ids, torch.int32, "tgt_ids"), V_draft, V_target, int(fallback),
                                         _ptr(d2t), _ptr(t2d), _stream(dev)), "sdv_tli_build_maps")
    return d2t, t2d


def sdv_tli_map_ids(table, ids, out=None):
    if out is None:
        out = torch.empty_like(ids, dtype=torch.int32)
    _check(_lib.lib().sdv_tli_map_ids(_ptr(table, torch.int32, "table"), table.numel(), _ptr(ids, torch.int32, "ids"),
                                      ids.numel(), _ptr(out, torch.int32, "out"), _stream(ids.device)),
           "sdv_tli_map_ids")
    return out


def sdv_tli_constrain_draft_logits(pruned, inter_ids, V_draft: int, full=None):
    B, K = pruned.shape
    if full is None:
        full = torch.empty((B, V_draft), dtype=torch.float32, device=pruned.device)
    _check(_lib.lib().sdv_tli_constrain_draft_logits(B, K, V_draft, _ptr(pruned, torch.float32, "pruned"),
                                                     _ptr(inter_ids, torch.int32, "inter_ids"),
                                                     _ptr(full, torch.float32, "full"), _stream(pruned.device)),
           "sdv_tli_constrain_draft_logits")
    return full


def sdv_tli_q_scatter(q_pruned, tgt_ids, V_target: int, q_target=None, ws=None):
    """tgt_ids None: reuse the inverse an earlier call left in ``ws``."""
    if tgt_ids is None and ws is None:
        raise ValueError("sdv_tli_q_scatter: tgt_ids=None reuses a workspace; pass the workspace of the call "
                         "that built the map")
    K = q_pruned.shape[-1]
    rows = math.prod(q_pruned.shape[:-1])             # also when K == 0
    dev = q_pruned.device
    if q_target is None:
        q_target = torch.empty(q_pruned.shape[:-1] + (V_target,), dtype=torch.float32, device=dev)
    L = _lib.lib()
    wp, wb = _workspace(L.sdv_tli_q_scatter_workspace_size(V_target), dev, ws)
    _check(L.sdv_tli_q_scatter(rows, K, V_target, _ptr(q_pruned, torch.float32, "q_pruned"),
                               _ptr(tgt_ids, torch.int32, "tgt_ids", allow_none=True),
                               _ptr(q_target, torch.float32, "q_target"),
                               wp, wb, _stream(dev)), "sdv_tli_q_scatter")
    return q_target
