"""The C ABI: the built library loads and exports every entry point that
include/sdv.h declares, and the binding declares each of them (no compute)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sdv.h")


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sdv_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_symbols()
    for must in ("sdv_draft_topk", "sdv_draft_topk_logits", "sdv_build_tree", "sdv_tree_verify_attention", "sdv_verify_accept",
                 "sdv_compact_kv", "sdv_tli_lm_head", "sdv_tli_map_ids", "sdv_tli_constrain_draft_logits",
                 "sdv_tli_q_scatter", "sdv_tli_build_maps", "sdv_draft_extend_prep", "sdv_build_chain", "sdv_kv_alloc_init",
                 "sdv_kv_alloc_backup", "sdv_kv_alloc_restore", "sdv_kv_alloc_free", "sdv_kv_alloc_extend",
                 "sdv_kv_alloc_branches", "sdv_kv_branch_pages", "sdv_last_error", "sdv_workspace_status",
                 "sdv_set_wait_limit", "sdv_tli_check", "sdv_softmax_rows"):
        assert must in names


def test_library_exports_every_declared_symbol():
    from speculative_decoding_eagle_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libsdv.so is not built; run `python -m speculative_decoding_eagle_amd.build`")
    lib = _lib.lib()
    for name in declared_symbols():
        assert hasattr(lib, name), name
        assert name in _lib.SIGNATURES, name
    assert lib.sdv_version() == 101
    assert lib.sdv_last_error() == b""


def test_host_side_validation_without_a_device():
    """Shape checks run on the host before anything is enqueued."""
    from speculative_decoding_eagle_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libsdv.so is not built")
    lib = _lib.lib()
    assert lib.sdv_draft_topk(None, 4, 10, 11, None, None, None, 0, None) == -2      # k > V
    assert b"k <= V" in lib.sdv_last_error()
    assert lib.sdv_draft_topk(None, 4, 100, 33, None, None, None, 0, None) == -3     # k above 32
    sh = _lib.TreeShape(2, 2, 3, 12)                                                  # N-1 = 11 > M = 10
    args = [None] * 15
    assert lib.sdv_build_tree(sh, *args, None) == -2
    assert lib.sdv_draft_topk(None, 0, 10, 2, None, None, None, 0, None) == 0         # empty is fine
    assert lib.sdv_draft_topk_logits(None, 2, 4, 10, 2, 1.0, None, None, None, 0, None) == -3   # unknown dtype
    assert lib.sdv_draft_topk_logits(None, 1, 4, 10, 2, 0.0, None, None, None, 0, None) == -2   # temperature 0
    assert lib.sdv_softmax_rows(None, 4, 10, 0.0, None, None) == -2      # temperature 0
    assert lib.sdv_softmax_rows(None, 4, 10, float("nan"), None, None) == -2
    assert lib.sdv_softmax_rows(None, 4, 0, 1.0, None, None) == -2        # V = 0
    assert lib.sdv_softmax_rows(None, -1, 10, 1.0, None, None) == -2
    assert lib.sdv_softmax_rows(None, 0, 10, 1.0, None, None) == 0        # nothing to do
    assert lib.sdv_softmax_rows(None, 4, 10, 1.0, None, None) == -1       # NULL
    assert lib.sdv_draft_topk_logits(None, 0, 4, 10, 11, 1.0, None, None, None, 0, None) == -2  # k > V
    ash = _lib.AttnShape(1, 4, 6, 4, 128, 1, 10, 10)                                  # Hq % Hkv != 0
    assert lib.sdv_tree_verify_attention(ash, ctypes.c_float(0.0), *([None] * 8), None, 0, None) == -2
    ash = _lib.AttnShape(1, 4, 8, 4, 96, 1, 10, 10)                                   # D not in {64,128}
    assert lib.sdv_tree_verify_attention(ash, ctypes.c_float(0.0), *([None] * 8), None, 0, None) == -3
    acc = _lib.AcceptShape(1, 4, 3, 100, 4, 7)                                        # unknown mode
    assert lib.sdv_verify_accept(acc, -1, *([None] * 14), None, 0, None) == -2
    assert lib.sdv_tli_lm_head(4, 100, 8, None, None, None, None) == -3               # H % 32 != 0


def test_tli_check_enforces_the_pages_validation_rules():
    """sglang PR #22883, "Modified files": TLI needs topk == 1 and
    num_draft_tokens == num_steps + 1; anything else is SDV_E_UNSUPPORTED."""
    from speculative_decoding_eagle_amd import _lib
    lib = _lib.lib()
    assert lib.sdv_tli_check(1, 4, 5) == 0
    assert lib.sdv_tli_check(1, 1, 2) == 0
    for k, S, N in [(8, 5, 64), (2, 4, 5), (1, 4, 4), (1, 4, 6), (1, 0, 1), (0, 4, 5)]:
        assert lib.sdv_tli_check(k, S, N) == -3, (k, S, N)
        assert b"TLI" in lib.sdv_last_error()
    import speculative_decoding_eagle_amd as sdv
    with pytest.raises(sdv.SdvError):
        sdv.sdv_tli_check(2, 4, 5)


def test_status_call_and_wait_limit_on_the_host():
    """Without a workspace the status is 0 and nothing touches a device; the
    wait limit is a host setting that round-trips."""
    from speculative_decoding_eagle_amd import _lib
    lib = _lib.lib()
    st = ctypes.c_uint32(7)
    assert lib.sdv_workspace_status(None, 0, ctypes.byref(st), 1, None) == 0 and st.value == 0
    assert lib.sdv_workspace_status(None, 4096, None, 1, None) == -1
    prev = lib.sdv_set_wait_limit(0)
    assert prev == 0xFFFFFFFF
    assert lib.sdv_set_wait_limit(0xFFFFFFFF) == 0
