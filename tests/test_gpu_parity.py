"""GPU parity: every stage of the HIP path against the CPU oracle on the same
seeded inputs.  Integer and index outputs must match bit for bit; attention
and the pruned LM head must lie within max |err| <= 2e-2 and
||err||_2 <= 1e-2 ||ref||_2."""
import sys

import numpy as np
import pytest
import torch

import speculative_decoding_eagle_amd as sdv
import workloads
from oracle import accept as oacc
from oracle import alloc as oal
from oracle import attention as oatt
from oracle import compact as ocmp
from oracle import extend as oext
from oracle import softmax as osm
from oracle import tli as otli
from oracle import topk as otopk
from oracle import tree as otree
from _helpers import (assert_attention_close, bf16_to_f64, dev, host, oracle_tree, plant_greedy,
                      plant_stochastic)

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    say("device", torch.cuda.get_device_name(0))
    yield
    torch.cuda.synchronize()


# ---------------------------------------------------------------------- A1

@pytest.mark.parametrize("rows,V,k,coarse", [(10, 1000, 2, False), (64, 4099, 8, False), (33, 128256, 8, False),
                                             (1100, 2048, 8, True), (200, 5000, 13, True), (5, 64, 32, True),
                                             (3, 7, 7, True), (1, 1, 1, False), (17, 40000, 4, True)])
def test_topk_bit_exact(rows, V, k, coarse):
    rng = np.random.default_rng(rows * 131 + V + k)
    if coarse:
        p = (rng.integers(0, 9, size=(rows, V)) / 16.0).astype(np.float32)   # many ties
    else:
        p = workloads.softmax_rows(rng.standard_normal((rows, V)).astype(np.float32) * 3)
    say("topk", rows, V, k)
    gp, gi = sdv.sdv_draft_topk(dev(p), k)
    torch.cuda.synchronize()
    op, oi = otopk.draft_topk(p, k)
    assert np.array_equal(host(gi), oi)
    assert np.array_equal(host(gp), op)


# Fused softmax + top-k from logits.  Ids must match bit for bit (the order
# is that of the logits); probabilities within 1e-4 relative: the exponent
# (x - m) * log2(e) / T rounds once in fp32 (|x - m| < 64 here: < 1e-5
# relative in p) and the normaliser sums about V / (256 * splits) terms per
# lane in fp32 before a fixed-order tree (< 512 * 2^-24 = 3e-5 relative).
@pytest.mark.parametrize("rows,V,k,T,bf16,kind", [
    (10, 1000, 2, 1.0, False, "normal"), (64, 4099, 8, 0.7, False, "normal"), (33, 128256, 8, 1.0, True, "normal"),
    (1056, 128256, 8, 1.0, True, "normal"), (300, 128256, 8, 0.7, False, "normal"), (5, 64, 32, 1.3, True, "ties"),
    (200, 5000, 13, 1.0, False, "ties"), (3, 7, 7, 2.0, True, "normal"), (1, 1, 1, 1.0, False, "normal"),
    (17, 40003, 4, 0.5, True, "masked"), (40, 9000, 16, 1.0, False, "masked"), (2, 131072, 32, 1.0, True, "ties"),
    (260, 90000, 8, 1.0, True, "normal"), (257, 100004, 16, 0.7, False, "ties")])
def test_topk_from_logits(rows, V, k, T, bf16, kind):
    rng = np.random.default_rng(rows * 7 + V + k)
    if kind == "ties":
        x = (rng.integers(-12, 4, size=(rows, V)) / 4.0).astype(np.float32)
    else:
        x = (rng.standard_normal((rows, V)) * 3.0).astype(np.float32)
    if kind == "masked":
        x[rng.random((rows, V)) < 0.9] = -np.inf
        x[:, 0] = 0.5                                          # every row keeps a finite entry
    if bf16:
        bits = workloads.to_bf16_bits(x)
        g = dev(bits).view(torch.bfloat16)
        ov, oi = otopk.draft_topk_from_logits(bits, k, T, bf16=True)
    else:
        g = dev(x)
        ov, oi = otopk.draft_topk_from_logits(x, k, T)
    say("topk_logits", rows, V, k, T, "bf16" if bf16 else "f32", kind)
    gp, gi = sdv.sdv_draft_topk_logits(g, k, T)
    torch.cuda.synchronize()
    assert np.array_equal(host(gi), oi)
    got = host(gp).astype(np.float64)
    assert np.all(np.abs(got - ov) <= 1e-4 * ov + 1e-37)


# Processed distributions softmax(logits / T).  The GPU computes in fp32
# (exponent 2^(x*c - m*c), c = log2(e)/T, normaliser summed in a fixed
# order); per entry its error against the float64 definition is the rounding
# of the exponent's argument, about |x - m| / T * 2^-23 relative (at most 60
# here, i.e. 7e-6), one ulp of the exponential, the normaliser's fp32 sum
# of up to a few hundred terms per thread (under 1e-5) and two roundings
# of the output: 3e-5 relative bounds it with room.  -inf entries are exact
# zeros.  Shapes: the vector path (V % 4 == 0) at the configs' V and rows,
# the scalar path (V % 4 != 0, V = 1), masked rows, several temperatures.
# Rows of 65536 to 135168 entries stay on chip between the passes (one
# workgroup per row, one per CU at a time): more rows than CUs (517, 300,
# 260), rows whose last register chunks lie past the row (V = 70004), the
# largest such row (135168, nine LDS chunks) next to the smallest read
# twice above it (135172), both sides of the lower end (65536, 65532), and
# rows that just fill the register chunks (98304) or add one float4 in LDS
# (98308).
@pytest.mark.parametrize("rows,V,T,kind", [
    (80, 128256, 1.0, "normal"), (24, 128256, 0.7, "normal"), (5, 128256, 0.5, "normal"), (7, 1000, 0.7, "normal"),
    (3, 5, 1.0, "normal"), (9, 4099, 2.0, "normal"), (4, 1, 1.0, "normal"), (6, 40000, 0.8, "masked"),
    (2, 131072, 1.0, "ties"), (0, 128256, 1.0, "normal"), (517, 70004, 0.9, "normal"),
    (300, 128256, 0.7, "masked"), (260, 135168, 1.0, "normal"), (7, 135172, 1.0, "normal"),
    (11, 65532, 1.0, "normal"), (13, 65536, 1.0, "ties"), (9, 98304, 1.0, "normal"), (9, 98308, 0.9, "normal")])
def test_softmax_rows_against_the_float64_definition(rows, V, T, kind):
    rng = np.random.default_rng(rows * 13 + V)
    if kind == "ties":
        x = (rng.integers(-12, 4, size=(rows, V)) / 4.0).astype(np.float32)
    else:
        x = (rng.standard_normal((rows, V)) * 3.0).astype(np.float32)
    if kind == "masked":
        x[rng.random((rows, V)) < 0.7] = -np.inf
        x[:, 0] = 0.5
    say("softmax_rows", rows, V, T, kind)
    got = sdv.sdv_softmax_rows(dev(x), T)
    again = sdv.sdv_softmax_rows(dev(x), T)
    torch.cuda.synchronize()
    g = host(got).astype(np.float64)
    assert np.array_equal(host(got), host(again))              # deterministic
    if rows == 0:
        return
    ref = osm.softmax_rows(x, T)
    assert np.all(np.abs(g - ref) <= 3e-5 * ref + 1e-37), float(np.max(np.abs(g - ref) / np.maximum(ref, 1e-37)))
    assert np.all(g[np.isneginf(x)] == 0.0)


# Rows beyond a multiple of the compute units are cut into equal pieces
# of the rows laid end to end: a row may be cut between workgroups, and one
# workgroup may hold the tail of one row and the head of the next.  Each row
# gets a group of equal values (its maximum, doubled) at random places, so
# its k best and their tie order straddle wherever the cuts fall; 2048 rows
# (a multiple of 256 compute units) take the one-workgroup-per-row path
# alone, 256, 512 and 768 rows (one to three per compute unit) are cut into
# four or two row-aligned pieces each, and V = 82020 and 100004 end in a
# partial window.
@pytest.mark.parametrize("rows,V,k", [(1056, 128256, 8), (300, 128256, 4), (2047, 4104, 8), (2048, 4104, 8),
                                      (5000, 4104, 2), (129, 65536, 16), (7, 9000, 32), (256, 128256, 1),
                                      (512, 128256, 8), (768, 65536, 4), (300, 82020, 8), (260, 100004, 3),
                                      (255, 128256, 8)])
def test_topk_segments(rows, V, k):
    rng = np.random.default_rng(rows * 17 + V + k)
    p = workloads.softmax_rows(rng.standard_normal((rows, V)).astype(np.float32) * 3)
    top = p.max(axis=1) * 2
    pos = rng.integers(0, V, size=(rows, k + 2))
    for r in range(rows):
        p[r, pos[r]] = top[r]
    say("topk segments", rows, V, k)
    gp, gi = sdv.sdv_draft_topk(dev(p), k)
    torch.cuda.synchronize()
    op, oi = otopk.draft_topk(p, k)
    assert np.array_equal(host(gi), oi)
    assert np.array_equal(host(gp), op)


# One workspace, zero-filled once, through calls of different shapes and
# both entry points: every call finds the row counters at zero and leaves
# them so (the counters sit at the start of the workspace).
def test_topk_workspace_reuse():
    lib = sdv._lib.lib()
    shapes = [(1056, 128256, 8, False), (64, 4099, 8, True), (5, 100000, 4, False), (1056, 128256, 8, True),
              (33, 128256, 8, False), (1056, 128256, 8, False)]
    need = max(max(lib.sdv_draft_topk_workspace_size(r, V, k), lib.sdv_draft_topk_logits_workspace_size(r, V, k))
               for r, V, k, _ in shapes)
    assert need > 0
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    cache = {}
    for rows, V, k, logits in shapes:
        key = (rows, V, k, logits)
        if key not in cache:
            rng = np.random.default_rng(rows + V + k)
            x = (rng.standard_normal((rows, V)) * 3.0).astype(np.float32)
            if logits:
                cache[key] = (x, otopk.draft_topk_from_logits(x, k, 1.0))
            else:
                p = workloads.softmax_rows(x)
                cache[key] = (p, otopk.draft_topk(p, k))
        x, (ov, oi) = cache[key]
        say("topk workspace reuse", rows, V, k, "logits" if logits else "probs")
        if logits:
            gp, gi = sdv.sdv_draft_topk_logits(dev(x), k, 1.0, ws=ws)
        else:
            gp, gi = sdv.sdv_draft_topk(dev(x), k, ws=ws)
        torch.cuda.synchronize()
        assert np.array_equal(host(gi), oi)
        got = host(gp).astype(np.float64)
        if logits:
            assert np.all(np.abs(got - ov) <= 1e-4 * ov + 1e-37)
        else:
            assert np.array_equal(host(gp), ov)
        assert not bool(ws[:65536].any()), "row counters left non-zero"


# -------------------------------------------------------------------- A2-A4

TREE_KEYS = ("tokens", "parent", "depth", "positions", "score", "q_row", "mask", "mask_bits", "retrieve_index",
             "next_token", "next_sibling")


def _gpu_tree(tp, ti, root, plen, k, S, N):
    t = sdv.sdv_build_tree(dev(tp), dev(ti), dev(root), dev(plen), k, S, N)
    torch.cuda.synchronize()
    out = {key: host(v) for key, v in t.items()}
    out["mask_bits"] = out["mask_bits"].view(np.uint32)
    return out


def _assert_tree_equal(g, o):
    for key in TREE_KEYS:
        assert np.array_equal(g[key], o[key].astype(g[key].dtype)), key


@pytest.mark.parametrize("name,V", [("c1", None), ("c2", 2000), ("c3", 3000), ("c4", 3000)])
def test_build_tree_bit_exact(name, V):
    cfg = workloads.get_config(name, **({"V": V} if V else {}))
    inp = workloads.generate(cfg, with_attention=False)
    say("build_tree", name, cfg.B, cfg.k, cfg.S, cfg.N)
    tp, ti = otopk.draft_topk(inp["draft_probs"], cfg.k)
    g = _gpu_tree(tp, ti, inp["root_token"], inp["prefix_len"], cfg.k, cfg.S, cfg.N)
    o = otree.build_tree(tp, ti, inp["root_token"], inp["prefix_len"], cfg.k, cfg.S, cfg.N)
    _assert_tree_equal(g, o)


# Tie-heavy scores over k from 1 to 32, pools up to 1056 entries; every
# kernel form (k rounded up to 1, 2, 4 or 8 with N - 1 <= 64 or above, and
# k > 8) appears.
@pytest.mark.parametrize("k,S,N", [(2, 3, 6), (3, 4, 30), (8, 5, 64), (4, 6, 85), (16, 2, 200), (1, 9, 10),
                                   (2, 1, 3), (5, 3, 1), (8, 5, 256), (7, 4, 100), (9, 3, 120), (32, 2, 256),
                                   (1, 80, 81), (2, 20, 70)])
def test_build_tree_ties_and_shapes(k, S, N):
    rng = np.random.default_rng(k * 100 + S * 10 + N)
    B = 5
    R = 1 + (S - 1) * k
    probs = (rng.integers(1, 9, size=(B, R, 40)) / 16.0).astype(np.float32)   # coarse -> score ties
    tp, ti = otopk.draft_topk(probs, k)
    root = rng.integers(0, 40, size=B).astype(np.int32)
    plen = rng.integers(0, 1000, size=B).astype(np.int32)
    say("build_tree ties", k, S, N)
    g = _gpu_tree(tp, ti, root, plen, k, S, N)
    o = otree.build_tree(tp, ti, root, plen, k, S, N)
    _assert_tree_equal(g, o)


# Top-k rows that are not sorted (columns shuffled) and rows with exact 0 and
# 1 entries: the builder may not assume the draft top-k's order.
@pytest.mark.parametrize("k,S,N,shuffle", [(8, 5, 64, True), (4, 4, 32, True), (3, 4, 30, True), (8, 5, 256, True),
                                           (2, 3, 6, True), (5, 3, 40, True), (1, 5, 6, True), (8, 5, 64, False),
                                           (4, 4, 32, False), (2, 20, 70, True), (1, 80, 81, False)])
def test_build_tree_unsorted_and_edge_rows(k, S, N, shuffle):
    rng = np.random.default_rng(k * 1000 + S * 100 + N + (7 if shuffle else 0))
    B = 6
    R = 1 + (S - 1) * k
    probs = (rng.integers(0, 17, size=(B, R, 64)) / 16.0).astype(np.float32)   # 0, 1/16, .., 1: ties, 0s and 1s
    tp, ti = otopk.draft_topk(probs, k)
    if shuffle:
        perm = np.argsort(rng.random((B, R, k)), axis=2)
        tp = np.take_along_axis(tp, perm, axis=2)
        ti = np.take_along_axis(ti, perm, axis=2)
    root = rng.integers(0, 64, size=B).astype(np.int32)
    plen = rng.integers(0, 1000, size=B).astype(np.int32)
    say("build_tree unsorted/edge", k, S, N, shuffle)
    g = _gpu_tree(np.ascontiguousarray(tp), np.ascontiguousarray(ti), root, plen, k, S, N)
    o = otree.build_tree(tp, ti, root, plen, k, S, N)
    _assert_tree_equal(g, o)


# Multi-layer draft chain: bit-exact against the oracle, then through the
# same accept kernels as the tree.
@pytest.mark.parametrize("B,S", [(1, 1), (7, 4), (300, 12), (3, 255)])
def test_build_chain_bit_exact(B, S):
    rng = np.random.default_rng(B * 1000 + S)
    tp = rng.random((B, S)).astype(np.float32)
    ti = rng.integers(0, 128256, size=(B, S)).astype(np.int32)
    root = rng.integers(0, 128256, size=B).astype(np.int32)
    plen = rng.integers(0, 50000, size=B).astype(np.int32)
    say("build chain", B, S)
    t = sdv.sdv_build_chain(dev(tp), dev(ti), dev(root), dev(plen))
    torch.cuda.synchronize()
    g = {key: host(v) for key, v in t.items()}
    g["mask_bits"] = g["mask_bits"].view(np.uint32)
    _assert_tree_equal(g, otree.build_chain(tp, ti, root, plen))


@pytest.mark.parametrize("planted", [False, True])
def test_chain_through_stochastic_accept(planted):
    """A k=1 workload (4 draft steps) drafted as a multi-layer chain: the
    GPU chain equals the oracle's, and the stochastic accept walk over it
    agrees bit for bit."""
    cfg = workloads.get_config("c2", V=3001)
    inp = workloads.generate(cfg, with_attention=False)
    tp, ti = otopk.draft_topk(inp["draft_probs"], 1)
    chain = otree.build_chain(tp, ti, inp["root_token"], inp["prefix_len"])
    say("chain accept", planted)
    t = sdv.sdv_build_chain(dev(tp), dev(ti), dev(inp["root_token"]), dev(inp["prefix_len"]))
    torch.cuda.synchronize()
    g = {key: host(v) for key, v in t.items()}
    g["mask_bits"] = g["mask_bits"].view(np.uint32)
    _assert_tree_equal(g, chain)
    p = inp["target"]
    if planted:
        p = plant_stochastic(p, inp["draft_probs"], chain, workloads.extra_rng(cfg, 7), cfg.S)
    ga = _gpu_accept(sdv.STOCHASTIC, chain, p, cfg.S, draft_probs=inp["draft_probs"], u_accept=inp["u_accept"],
                     u_draw=inp["u_draw"])
    o = oacc.verify_stochastic(chain, p, inp["draft_probs"], inp["u_accept"], inp["u_draw"], cfg.S)
    _assert_accept_equal(ga, o)
    if planted:
        assert o["accept_len"].max() > 0


# -------------------------------------------------------------------- A6-A7

def _gpu_accept(mode, tree, target, S, **kw):
    gt = {key: dev(tree[key]) for key in ("tokens", "next_token", "next_sibling", "q_row")}
    args = {}
    for key in ("draft_probs", "u_accept", "u_draw", "remaining"):
        if kw.get(key) is not None:
            args[key] = dev(kw[key])
    if kw.get("ws") is not None:
        args["ws"] = kw["ws"]
    r = sdv.sdv_verify_accept(mode, gt, dev(target), S, eos_id=kw.get("eos_id", -1), **args)
    torch.cuda.synchronize()
    return {key: host(v) for key, v in r.items()}


def _assert_accept_equal(g, o):
    for key in ("accept_len", "accept_path", "commit_tokens", "commit_len", "next_root"):
        assert np.array_equal(g[key], o[key]), key


@pytest.mark.parametrize("name,V,planted", [("c1", None, False), ("c1", None, True), ("c3", 5000, True),
                                            ("c3", 128256, True), ("c4", 4097, True)])
def test_accept_greedy_bit_exact(name, V, planted):
    cfg = workloads.get_config(name, **({"V": V} if V else {}))
    if name == "c3" and V == 128256:
        cfg = cfg.replace(B=8)
    inp = workloads.generate(cfg, with_attention=False)
    tree = oracle_tree(inp, cfg)
    target = inp["target"]          # stochastic configs: the p rows serve as logits
    if planted:
        target = plant_greedy(target, tree, workloads.extra_rng(cfg, 1), cfg.S)
    say("accept greedy", name, cfg.B, cfg.V, planted)
    g = _gpu_accept(sdv.GREEDY, tree, target, cfg.S)
    o = oacc.verify_greedy(tree, target, cfg.S)
    _assert_accept_equal(g, o)
    if planted and cfg.B >= 8:
        assert o["accept_len"].max() > 0


def test_accept_greedy_budget_and_eos():
    cfg = workloads.get_config("c3", V=3000, B=12)
    inp = workloads.generate(cfg, with_attention=False)
    tree = oracle_tree(inp, cfg)
    rng = workloads.extra_rng(cfg, 2)
    target = plant_greedy(inp["target"], tree, rng, cfg.S)
    remaining = rng.integers(0, 4, size=cfg.B).astype(np.int32)
    say("accept greedy budget")
    g = _gpu_accept(sdv.GREEDY, tree, target, cfg.S, remaining=remaining)
    _assert_accept_equal(g, oacc.verify_greedy(tree, target, cfg.S, remaining=remaining))
    o0 = oacc.verify_greedy(tree, target, cfg.S)
    eos = int(o0["commit_tokens"][0, 0])
    say("accept greedy eos", eos)
    g = _gpu_accept(sdv.GREEDY, tree, target, cfg.S, eos_id=eos)
    _assert_accept_equal(g, oacc.verify_greedy(tree, target, cfg.S, eos_id=eos))


@pytest.mark.parametrize("name,V,B,planted", [("c2", None, None, False), ("c2", 3001, None, True),
                                              ("c4", 4096, 16, False), ("c4", 4096, 16, True),
                                              ("c4", 128256, 8, True), ("c1", None, None, True)])
def test_accept_stochastic_bit_exact(name, V, B, planted):
    over = {}
    if V:
        over["V"] = V
    if B:
        over["B"] = B
    cfg = workloads.get_config(name, **over)
    if cfg.mode != "stochastic":
        cfg = cfg.replace(mode="stochastic")
    inp = workloads.generate(cfg, with_attention=False)
    tree = oracle_tree(inp, cfg)
    p = inp["target"]
    if planted:
        p = plant_stochastic(p, inp["draft_probs"], tree, workloads.extra_rng(cfg, 3), cfg.S)
    say("accept stochastic", name, cfg.B, cfg.V, planted)
    g = _gpu_accept(sdv.STOCHASTIC, tree, p, cfg.S, draft_probs=inp["draft_probs"], u_accept=inp["u_accept"],
                    u_draw=inp["u_draw"])
    o = oacc.verify_stochastic(tree, p, inp["draft_probs"], inp["u_accept"], inp["u_draw"], cfg.S)
    _assert_accept_equal(g, o)


_FULL_ACCEPT = {}


def _full_accept_inputs(name):
    """Inputs and oracle tree of a workload at its full batch and vocabulary
    (the launch configuration the bench times), made once per module."""
    if name not in _FULL_ACCEPT:
        cfg = workloads.get_config(name)
        inp = workloads.generate(cfg, with_attention=False)
        _FULL_ACCEPT[name] = (cfg, inp, oracle_tree(inp, cfg))
    return _FULL_ACCEPT[name]


# The accept walk at the workloads' own sizes: c3 greedy (32 requests, one
# group of 8 workgroups each, 64 floats per thread) and c4 rejection
# sampling (64 requests), literal and with planted acceptance.
@pytest.mark.parametrize("name,planted", [("c3", False), ("c3", True), ("c4", False), ("c4", True)])
def test_accept_full_config(name, planted):
    cfg, inp, tree = _full_accept_inputs(name)
    say("accept full", name, cfg.B, cfg.V, cfg.mode, planted)
    if cfg.mode == "greedy":
        target = inp["target"]
        if planted:
            target = plant_greedy(target, tree, workloads.extra_rng(cfg, 1), cfg.S)
        g = _gpu_accept(sdv.GREEDY, tree, target, cfg.S)
        o = oacc.verify_greedy(tree, target, cfg.S)
    else:
        p = inp["target"]
        if planted:
            p = plant_stochastic(p, inp["draft_probs"], tree, workloads.extra_rng(cfg, 3), cfg.S)
        g = _gpu_accept(sdv.STOCHASTIC, tree, p, cfg.S, draft_probs=inp["draft_probs"], u_accept=inp["u_accept"],
                        u_draw=inp["u_draw"])
        o = oacc.verify_stochastic(tree, p, inp["draft_probs"], inp["u_accept"], inp["u_draw"], cfg.S)
    _assert_accept_equal(g, o)
    if planted:
        assert o["accept_len"].sum() > 0


def test_accept_leaves_its_workspace_zero():
    """The exchange words and counters are cleared by each call's last
    workgroup per request: one explicit zero-filled workspace serves calls
    of both modes and several batch sizes, and is all zero after each."""
    cfg = workloads.get_config("c4", V=4096, B=16)
    inp = workloads.generate(cfg, with_attention=False)
    tree = oracle_tree(inp, cfg)
    p = plant_stochastic(inp["target"], inp["draft_probs"], tree, workloads.extra_rng(cfg, 8), cfg.S)
    ws = torch.zeros(1 << 20, dtype=torch.uint8, device="cuda")
    say("accept workspace reset")
    for sub in (16, 5, 16):
        t = {key: v[:sub] for key, v in tree.items()}
        g = _gpu_accept(sdv.STOCHASTIC, t, p[:sub], cfg.S, draft_probs=inp["draft_probs"][:sub],
                        u_accept=inp["u_accept"][:sub], u_draw=inp["u_draw"][:sub], ws=ws)
        _assert_accept_equal(g, oacc.verify_stochastic(t, p[:sub], inp["draft_probs"][:sub], inp["u_accept"][:sub],
                                                       inp["u_draw"][:sub], cfg.S))
        assert int(torch.count_nonzero(ws)) == 0
        g = _gpu_accept(sdv.GREEDY, t, p[:sub], cfg.S, ws=ws)
        _assert_accept_equal(g, oacc.verify_greedy(t, p[:sub], cfg.S))
        assert int(torch.count_nonzero(ws)) == 0


def test_accept_stochastic_degenerate_rows():
    """A leaf row with zero mass takes the argmax; tiny masses below 2^-40 too."""
    cfg = workloads.get_config("c2", V=1000, B=4)
    inp = workloads.generate(cfg, with_attention=False)
    tree = oracle_tree(inp, cfg)
    p = plant_stochastic(inp["target"], inp["draft_probs"], tree, workloads.extra_rng(cfg, 4), cfg.S)
    # every node accepted up to the leaf, whose row is (nearly) empty
    for b in range(cfg.B):
        u = 0
        while tree["next_token"][b, u] >= 0:
            p[b, u] = inp["draft_probs"][b, tree["q_row"][b, u]]
            u = tree["next_token"][b, u]
        p[b, u] = 0.0
        if b % 2:
            p[b, u, 17 + b] = np.float32(2.0 ** -45)
    say("accept stochastic degenerate")
    g = _gpu_accept(sdv.STOCHASTIC, tree, p, cfg.S, draft_probs=inp["draft_probs"], u_accept=inp["u_accept"],
                    u_draw=inp["u_draw"])
    o = oacc.verify_stochastic(tree, p, inp["draft_probs"], inp["u_accept"], inp["u_draw"], cfg.S)
    _assert_accept_equal(g, o)


# ---------------------------------------------------------------------- A8

def _accept_paths(rng, B, N, S, tree=None):
    acc_len = np.zeros(B, np.int32)
    acc_path = np.full((B, S + 1), -1, np.int32)
    for b in range(B):
        a = int(rng.integers(0, min(S, N - 1) + 1))
        path = [0] + sorted(rng.choice(np.arange(1, N), size=a, replace=False).tolist())
        acc_len[b] = a
        acc_path[b, :a + 1] = path
    return acc_len, acc_path


# The last case is c4's own shape: 64 requests, page 16, 8 KV heads of 128
# (2 KB per token and pool), prefixes of 1024 to 8192 tokens; its pools hold
# a position pattern instead of random bits (600 MB each).
@pytest.mark.parametrize("page,layers,B,N,S,Hkv,D,Lmax", [
    (1, 1, 6, 12, 4, 2, 16, 300), (1, 1, 32, 64, 5, 2, 16, 300), (16, 3, 9, 32, 4, 2, 16, 300),
    (4, 2, 7, 12, 6, 2, 16, 300), (16, 1, 64, 32, 4, 2, 16, 300), (8, 2, 5, 256, 9, 2, 16, 300),
    (16, 1, 64, 32, 4, 8, 128, 8192)])
def test_compaction_bit_exact(page, layers, B, N, S, Hkv, D, Lmax):
    rng = np.random.default_rng(page * 1000 + layers * 100 + N)
    big = Lmax > 300
    L = rng.integers(1024 if big else 0, Lmax + (1 if big else 0), size=B).astype(np.int32)
    need = (L + N + page - 1) // page
    total = int(need.sum()) + 5
    perm = rng.permutation(total).astype(np.int32)
    table = np.full((B, int(need.max()) + 2), -1, np.int32)
    off = 0
    for b in range(B):
        table[b, :need[b]] = perm[off:off + need[b]]
        off += need[b]
    if big:
        pattern = (np.arange(total * page * Hkv * D, dtype=np.uint32) * np.uint32(40503) % np.uint32(65521)).astype(np.uint16)
        kps = [pattern.reshape(total * page, Hkv, D) for _ in range(layers)]
        vps = [(pattern ^ np.uint16(0x5A5A)).reshape(total * page, Hkv, D) for _ in range(layers)]
    else:
        kps = [rng.integers(0, 65535, size=(total * page, Hkv, D)).astype(np.uint16) for _ in range(layers)]
        vps = [rng.integers(0, 65535, size=(total * page, Hkv, D)).astype(np.uint16) for _ in range(layers)]
    a, path = _accept_paths(rng, B, N, S)
    say("compact", page, layers, B, N, S, Hkv, D, Lmax)
    gt = dev(table)
    gk = [dev(x) for x in kps] if page > 1 else []
    gv = [dev(x) for x in vps] if page > 1 else []
    new_len, freed, nf = sdv.sdv_compact_kv(gt, dev(L), dev(a), dev(path), N, S, page, gk, gv)
    torch.cuda.synchronize()
    t2, k2, v2, nl, fr = ocmp.compact_kv(table, kps, vps, L, a, path, N, page)
    assert np.array_equal(host(gt), t2)
    assert np.array_equal(host(new_len), nl)
    n = int(host(nf)[0])
    assert n == len(fr)
    assert np.array_equal(host(freed)[:n], fr)
    if page > 1:
        for x, y in zip(gk + gv, k2 + v2):
            assert np.array_equal(host(x).view(np.uint16), y)


# ------------------------------------------------------- KV allocation

def _alloc_equal(g, o):
    torch.cuda.synchronize()
    st = host(g.state)
    assert st[:3].tolist() == [o.top, o.pushes, o.error]
    assert np.array_equal(host(g.free_ids)[:o.capacity], o.free_ids)


def _alloc_pair(capacity):
    """A fresh GPU allocator and its oracle twin."""
    g = sdv.sdv_kv_alloc_init(capacity)
    o = oal.KVAllocator(capacity)
    return g, o


@pytest.mark.parametrize("B,topk,S", [(5, 4, 3), (1, 1, 1), (300, 8, 5), (8191, 2, 3), (8192, 1, 1)])
def test_kv_alloc_page1_draft_and_rollback(B, topk, S):
    cap = B * topk * S + 77
    g, o = _alloc_pair(cap)
    seq = np.random.default_rng(B).integers(0, 500, size=B).astype(np.int32)
    table = np.zeros((B, 1), np.int32)
    say("kv alloc page 1", B, topk, S)
    bk = sdv.sdv_kv_alloc_backup(g)
    obk = o.backup()
    gp, gl = sdv.sdv_kv_alloc_branches(g, 1, topk, S, dev(table), dev(seq))
    op, ol, _, _ = oal.alloc_branches(o, table, seq, topk, S, 1)
    _alloc_equal(g, o)
    assert np.array_equal(host(gp), op) and np.array_equal(host(gl), ol)
    sdv.sdv_kv_alloc_restore(g, bk)
    o.restore(obk)
    _alloc_equal(g, o)
    assert o.top == cap and o.error == 0


@pytest.mark.parametrize("P,topk,S", [(4, 3, 3), (16, 4, 5), (16, 8, 20), (8, 2, 9)])
def test_kv_alloc_duplicated_partial_pages(P, topk, S):
    """Branch layout with the partial-page copies, every layer, K and V."""
    rng = np.random.default_rng(P * 100 + topk * 10 + S)
    B, layers, Hkv, D = 6, 3, 2, 64
    cap = 400
    g, o = _alloc_pair(cap)
    seq = rng.integers(0, 5 * P, size=B).astype(np.int32)
    seq[0] = 2 * P                                          # page aligned: no copy
    max_pages = 8
    table = np.full((B, max_pages), -1, np.int32)
    gt = dev(table)
    sdv.sdv_kv_alloc_extend(g, P, 0, gt, dev(np.zeros(B, np.int32)))      # n = 0: nothing taken
    table, _ = oal.alloc_extend(o, table, np.zeros(B, np.int32), 0, P)
    gt = dev(table)
    gseq0 = dev(np.zeros(B, np.int32))
    sdv.sdv_kv_alloc_extend(g, P, int(seq.max()), gt, gseq0)               # give every request pages
    table, _ = oal.alloc_extend(o, table, np.zeros(B, np.int32), int(seq.max()), P)
    _alloc_equal(g, o)
    assert np.array_equal(host(gt), table)
    slots = cap * P
    kp = [rng.integers(0, 65536, size=(slots, Hkv, D)).astype(np.uint16) for _ in range(layers)]
    vp = [rng.integers(0, 65536, size=(slots, Hkv, D)).astype(np.uint16) for _ in range(layers)]
    gk, gv = [dev(x) for x in kp], [dev(x) for x in vp]
    say("kv alloc branches", P, topk, S)
    gp, gl = sdv.sdv_kv_alloc_branches(g, P, topk, S, gt, dev(seq), gk, gv)
    op, ol, ok2, ov2 = oal.alloc_branches(o, table, seq, topk, S, P, kp, vp)
    _alloc_equal(g, o)
    assert np.array_equal(host(gp), op) and np.array_equal(host(gl), ol)
    for a, b in zip(gk + gv, ok2 + ov2):
        assert np.array_equal(host(a).view(np.uint16), b)


@pytest.mark.parametrize("P,n", [(1, 7), (4, 5), (16, 64), (16, 1)])
def test_kv_alloc_extend(P, n):
    rng = np.random.default_rng(P + n)
    B, max_pages, cap = 40, 64, 3000
    g, o = _alloc_pair(cap)
    seq = np.zeros(B, np.int32)
    table = np.full((B, max_pages), -1, np.int32)
    gt = dev(table)
    say("kv alloc extend", P, n)
    for _ in range(3):
        grow = rng.integers(0, 3, size=B).astype(np.int32) * n // 2
        gl = sdv.sdv_kv_alloc_extend(g, P, n, gt, dev(seq))
        table, ol = oal.alloc_extend(o, table, seq, n, P)
        _alloc_equal(g, o)
        assert np.array_equal(host(gt), table) and np.array_equal(host(gl), ol)
        seq = seq + np.minimum(grow, n).astype(np.int32)


def test_kv_alloc_errors_change_nothing():
    g, o = _alloc_pair(10)
    table = np.full((2, 4), -1, np.int32)
    gt = dev(table)
    say("kv alloc errors")
    gl = sdv.sdv_kv_alloc_extend(g, 1, 6, gt, dev(np.zeros(2, np.int32)))          # 12 > 10
    t2, ol = oal.alloc_extend(o, table, np.zeros(2, np.int32), 6, 1)
    _alloc_equal(g, o)
    assert (host(gl) == -1).all() and np.array_equal(host(gt), table) and o.error == 1
    gp, gl = sdv.sdv_kv_alloc_branches(g, 1, 3, 4, gt, dev(np.zeros(2, np.int32)))  # 24 > 10
    oal.alloc_branches(o, table, np.zeros(2, np.int32), 3, 4, 1)
    _alloc_equal(g, o)
    assert (host(gp) == -1).all() and (host(gl) == -1).all()
    bk, obk = sdv.sdv_kv_alloc_backup(g), o.backup()
    sdv.sdv_kv_alloc_extend(g, 1, 2, gt, dev(np.zeros(2, np.int32)))
    table, _ = oal.alloc_extend(o, table, np.zeros(2, np.int32), 2, 1)
    ids = np.array([table[0, 0]], np.int32)
    sdv.sdv_kv_alloc_free(g, dev(ids), dev(np.array([1], np.int32)))
    o.push(ids)
    sdv.sdv_kv_alloc_restore(g, bk)                                                  # refused: a push since
    o.restore(obk)
    _alloc_equal(g, o)
    assert o.error & 2
    many = np.arange(20, dtype=np.int32)
    sdv.sdv_kv_alloc_free(g, dev(many), dev(np.array([20], np.int32)))               # overflow
    o.push(many)
    _alloc_equal(g, o)
    assert o.error & 4


@pytest.mark.parametrize("page", [1, 4])
def test_kv_alloc_speculative_rounds_with_compaction(page):
    """Rounds of: backup, draft branches, rollback, verify-tree extend,
    compaction (GPU and oracle each on their own state), release of the freed
    units.  The allocator, tables and pools agree after every round."""
    rng = np.random.default_rng(page)
    B, N, S, topk = 8, 12, 4, 3
    Hkv, D, layers = 2, 64, 2
    max_pages = 256 // page
    cap = B * max_pages
    g, o = _alloc_pair(cap)
    seq = rng.integers(1, 40, size=B).astype(np.int32)
    table = np.full((B, max_pages), -1, np.int32)
    gt = dev(table)
    sdv.sdv_kv_alloc_extend(g, page, int(seq.max()), gt, dev(np.zeros(B, np.int32)))
    table, _ = oal.alloc_extend(o, table, np.zeros(B, np.int32), int(seq.max()), page)
    # page 1 moves no KV bytes (slot maps only); page 4 copies partial pages
    # and compacts rows in the pools
    nl = layers if page > 1 else 0
    kp = [rng.integers(0, 65536, size=(cap * page, Hkv, D)).astype(np.uint16) for _ in range(nl)]
    vp = [rng.integers(0, 65536, size=(cap * page, Hkv, D)).astype(np.uint16) for _ in range(nl)]
    gk, gv = [dev(x) for x in kp], [dev(x) for x in vp]
    gseq = dev(seq)
    for rnd in range(4):
        say("kv alloc round", page, rnd)
        bk, obk = sdv.sdv_kv_alloc_backup(g), o.backup()
        gp, gl = sdv.sdv_kv_alloc_branches(g, page, topk, S, gt, gseq, gk, gv)
        op, ol, kp, vp = oal.alloc_branches(o, table, seq, topk, S, page, kp, vp)
        assert np.array_equal(host(gp), op) and np.array_equal(host(gl), ol)
        sdv.sdv_kv_alloc_restore(g, bk)
        o.restore(obk)
        sdv.sdv_kv_alloc_extend(g, page, N, gt, gseq)
        table, _ = oal.alloc_extend(o, table, seq, N, page)
        _alloc_equal(g, o)
        acc = rng.integers(0, S + 1, size=B).astype(np.int32)
        path = np.full((B, S + 1), -1, np.int32)
        for b in range(B):
            path[b, :acc[b] + 1] = np.sort(np.concatenate([[0], rng.choice(np.arange(1, N), acc[b], replace=False)]))
        new_len, freed, num_freed = sdv.sdv_compact_kv(gt, gseq, dev(acc), dev(path), N, S, page, gk, gv)
        table, kp, vp, onew, ofreed = ocmp.compact_kv(table, kp, vp, seq, acc, path, N, page)
        sdv.sdv_kv_alloc_free(g, freed, num_freed)
        o.push(ofreed)
        _alloc_equal(g, o)
        assert np.array_equal(host(gt), table) and np.array_equal(host(new_len), onew)
        for a, b in zip(gk + gv, kp + vp):
            assert np.array_equal(host(a).view(np.uint16), b)
        seq = onew.astype(np.int32)
        gseq = new_len
        assert o.error == 0


# ------------------------------------------------- draft extend index prep

def _extend_case(prefix_len, commit_len, commit_tokens, accept_path, N, t2d=None):
    B = commit_tokens.shape[0]
    g = sdv.sdv_draft_extend_prep(dev(prefix_len.astype(np.int32)), dev(commit_len.astype(np.int32)),
                                  dev(commit_tokens.astype(np.int32)), dev(accept_path.astype(np.int32)), N,
                                  t2d=None if t2d is None else dev(t2d))
    torch.cuda.synchronize()
    o = oext.draft_extend_prep(prefix_len, commit_len, commit_tokens, accept_path, N, t2d=t2d)
    total = int(o["extend_start"][-1])
    assert np.array_equal(host(g["extend_start"]), o["extend_start"])
    for key in ("input_ids", "positions", "hidden_index"):
        assert np.array_equal(host(g[key])[:total], o[key]), key
    for key in ("last_index", "seq_len"):
        assert np.array_equal(host(g[key]), o[key]), key
    assert B == 0 or total <= B * commit_tokens.shape[1]


@pytest.mark.parametrize("seed,tli", [(0, False), (1, True)])
def test_extend_prep_after_accept(seed, tli):
    """The accept walk's outputs (oracle, on a c3-shaped tree with planted
    acceptance and budgets) through the GPU and oracle index preparation."""
    cfg = workloads.get_config("c3", V=3000, B=24)
    inp = workloads.generate(cfg, with_attention=False)
    tree = oracle_tree(inp, cfg)
    rng = np.random.default_rng(seed)
    target = plant_greedy(inp["target"], tree, rng, cfg.S)
    rem = rng.integers(0, cfg.S + 2, size=cfg.B).astype(np.int32)
    r = oacc.verify_greedy(tree, target, cfg.S, remaining=rem)
    t2d = None
    if tli:
        K = 1200
        inter = np.sort(rng.choice(4000, K, replace=False)).astype(np.int32)
        tgt = rng.choice(cfg.V, K, replace=False).astype(np.int32)
        t2d = otli.build_maps(inter, tgt, 4000, cfg.V, int(np.setdiff1d(np.arange(4000), inter)[0]))[1]
    say("extend prep after accept", seed, tli)
    _extend_case(inp["prefix_len"], r["commit_len"], r["commit_tokens"], r["accept_path"], cfg.N, t2d)


@pytest.mark.parametrize("B,S,N", [(0, 4, 8), (1, 0, 1), (37, 5, 64), (1500, 4, 32), (3000, 63, 256)])
def test_extend_prep_shapes(B, S, N):
    """Synthetic batches: empty, single, several scan chunks, the largest S;
    about a fifth of the requests commit nothing."""
    rng = np.random.default_rng(B + S)
    S1 = S + 1
    commit_len = np.where(rng.random(B) < 0.2, 0, rng.integers(1, S1 + 1, size=B)).astype(np.int32)
    tokens = np.full((B, S1), -1, np.int32)
    path = np.full((B, S1), -1, np.int32)
    for b in range(B):
        c = commit_len[b]
        tokens[b, :c] = rng.integers(0, 50000, size=c)
        path[b, :c] = np.sort(rng.choice(N, size=c, replace=False)) if c <= N else 0
    prefix = rng.integers(0, 100000, size=B).astype(np.int32)
    t2d = rng.integers(0, 30000, size=50000).astype(np.int32)
    say("extend prep shapes", B, S, N)
    _extend_case(prefix, commit_len, tokens, path, N)
    _extend_case(prefix, commit_len, tokens, path, N, t2d)


def test_extend_prep_clamps_out_of_range_inputs():
    """Documented handling of inputs outside the contract: commit lengths are
    clamped into [0, S+1]; bad tokens and nodes give -1 in their row."""
    S, N = 3, 6
    commit_len = np.array([9, -2, 2, 4], np.int32)
    tokens = np.array([[1, 2, 3, 4], [5, 6, 7, 8], [-5, 70, 0, 0], [1, 2, 3, 4]], np.int32)
    path = np.array([[0, 1, 2, 3], [0, 1, 2, 3], [0, 9, 0, 0], [0, 1, 2, 3]], np.int32)
    prefix = np.array([10, 20, 30, 40], np.int32)
    t2d = np.arange(60, dtype=np.int32) * 2
    say("extend prep clamps")
    g = sdv.sdv_draft_extend_prep(dev(prefix), dev(commit_len), dev(tokens), dev(path), N, t2d=dev(t2d))
    torch.cuda.synchronize()
    assert host(g["extend_start"]).tolist() == [0, 4, 4, 6, 10]
    assert host(g["input_ids"])[:10].tolist() == [2, 4, 6, 8, -1, -1, 2, 4, 6, 8]
    assert host(g["hidden_index"])[:10].tolist() == [0, 1, 2, 3, 12, -1, 18, 19, 20, 21]
    assert host(g["positions"])[:10].tolist() == [11, 12, 13, 14, 31, 32, 41, 42, 43, 44]
    assert host(g["last_index"]).tolist() == [3, -1, 5, 9]
    assert host(g["seq_len"]).tolist() == [15, 21, 33, 45]


# ---------------------------------------------------------------------- A5

def _attn_case(cfg, inp, requests=None, want_lse=True, split_keys=True):
    t = oracle_tree(inp, cfg)
    W = (cfg.N + 31) // 32
    say("attention", cfg.name, cfg.B, cfg.N, cfg.Hq, cfg.Hkv, cfg.D, cfg.page, "split" if split_keys else "whole")
    out, lse = sdv.sdv_tree_verify_attention(dev(inp["q"]), dev(inp["k_pool"]), dev(inp["v_pool"]),
                                             dev(inp["page_table"]), dev(inp["prefix_len"]),
                                             dev(t["mask_bits"].view(np.int32)), page=cfg.page, want_lse=want_lse,
                                             split_keys=split_keys)
    torch.cuda.synchronize()
    assert t["mask_bits"].shape[-1] == W
    ro, rl = oatt.tree_verify_attention(inp["q"], inp["k_pool"], inp["v_pool"], inp["page_table"],
                                        inp["prefix_len"], t["mask"], page=cfg.page, requests=requests)
    got = bf16_to_f64(out)
    sel = list(range(cfg.B)) if requests is None else list(requests)
    assert_attention_close(got[sel], ro[sel])
    if want_lse:
        # lse = m + log(l); the row sum l adds the bf16-rounded weights the PV
        # product uses, each within bf16's unit roundoff 2^-8 of the exact
        # weight, so |d lse| <= 2^-8 (+ fp32 rounding): 4e-3.
        assert np.abs(host(lse)[sel] - rl[sel]).max() < 4e-3


def test_attention_c1_full():
    cfg = workloads.get_config("c1")
    _attn_case(cfg, workloads.generate(cfg))


@pytest.mark.parametrize("over", [dict(B=3, L_min=100, L_max=300), dict(B=2, N=13, Hq=6, Hkv=2, D=64, L_min=1, L_max=70),
                                  dict(B=2, N=40, Hq=8, Hkv=8, D=128, L_min=0, L_max=0),
                                  dict(B=2, N=256, k=8, S=6, Hq=4, Hkv=1, D=64, L_min=30, L_max=90)])
def test_attention_small_shapes(over):
    cfg = workloads.get_config("c3", V=256, **over)
    _attn_case(cfg, workloads.generate(cfg))


def test_attention_paged_small():
    cfg = workloads.get_config("c4", V=256, B=3, L_min=40, L_max=200)
    _attn_case(cfg, workloads.generate(cfg))


def _attn_gpu(cfg, inp, t, split_keys):
    say("attention", cfg.name, cfg.B, cfg.N, cfg.Hq, cfg.Hkv, cfg.D, cfg.page, "split" if split_keys else "whole")
    out, lse = sdv.sdv_tree_verify_attention(dev(inp["q"]), dev(inp["k_pool"]), dev(inp["v_pool"]),
                                             dev(inp["page_table"]), dev(inp["prefix_len"]),
                                             dev(t["mask_bits"].view(np.int32)), page=cfg.page, want_lse=True,
                                             split_keys=split_keys)
    torch.cuda.synchronize()
    return bf16_to_f64(out), host(lse)


@pytest.mark.parametrize("name", ["c3", "c4"])
def test_attention_full_config_every_request(name):
    """The workloads' own shapes, every request (c3: 32 units of 256 rows with
    the longest-first ranking, the XCD dealing and the key split; c4: 64
    requests of 514 pages at most), with and without the key split."""
    cfg = workloads.get_config(name, V=256)
    inp = workloads.generate(cfg)
    t = oracle_tree(inp, cfg)
    ro, rl = oatt.tree_verify_attention(inp["q"], inp["k_pool"], inp["v_pool"], inp["page_table"],
                                        inp["prefix_len"], t["mask"], page=cfg.page)
    for split in (True, False):
        got, lse = _attn_gpu(cfg, inp, t, split)
        assert_attention_close(got, ro)
        assert np.abs(lse - rl).max() < 4e-3


def test_attention_c3_tree_keys_carry_the_output():
    """c3's shape with every prefix V row zero: each output row is then made of
    its node's own visible tree keys only (depth + 1 of them), so a single wrong
    mask bit moves that row by a large fraction of itself.  Checked row by row
    (relative to the row's norm) on every request, split and unsplit."""
    cfg = workloads.get_config("c3", V=256)
    inp = workloads.generate(cfg)
    t = oracle_tree(inp, cfg)
    keep = np.zeros(inp["v_pool"].shape[0], bool)
    for b in range(cfg.B):
        L = int(inp["prefix_len"][b])
        keep[oatt.slot_of(inp["page_table"], b, np.arange(L, L + cfg.N), cfg.page)] = True
    v = inp["v_pool"].copy()
    v[~keep] = 0
    inp = dict(inp, v_pool=v)
    ro, _ = oatt.tree_verify_attention(inp["q"], inp["k_pool"], inp["v_pool"], inp["page_table"],
                                       inp["prefix_len"], t["mask"], page=cfg.page)
    ref_rows = ro.reshape(-1, cfg.D)
    nrm = np.linalg.norm(ref_rows, axis=1)
    assert nrm.min() > 0
    for split in (True, False):
        got, _ = _attn_gpu(cfg, inp, t, split)
        assert_attention_close(got, ro)
        rel = np.linalg.norm(got.reshape(-1, cfg.D) - ref_rows, axis=1) / nrm
        # bf16 weights and output: a few 2^-9 relative per row; one wrong
        # mask bit moves a row by about 1 / sqrt(depth + 1) of itself
        assert rel.max() < 3e-2, "row %d off by %.3g of its norm" % (int(np.argmax(rel)), rel.max())


# More than 128 query rows per (request, KV head): the wide kernel, with and
# without the key split.
_WIDE = [dict(B=3, L_min=100, L_max=300),                                     # 256 rows, G=4
         dict(B=2, N=64, Hq=8, Hkv=2, D=64, L_min=200, L_max=700),           # D=64
         dict(B=4, N=100, Hq=6, Hkv=2, D=128, L_min=0, L_max=5),             # 300 rows (G=3): row blocks split nodes
         dict(B=3, N=20, Hq=16, Hkv=1, D=128, L_min=1, L_max=64),            # G=16, one or two tiles in all
         dict(B=2, N=33, Hq=32, Hkv=4, D=128, page=16, L_min=60, L_max=900),  # paged
         dict(B=1, N=64, Hq=4, Hkv=1, D=128, L_min=9000, L_max=9000)]        # page-window refreshes in each chunk


@pytest.mark.parametrize("over", _WIDE)
@pytest.mark.parametrize("split", [True, False])
def test_attention_wide_shapes(over, split):
    cfg = workloads.get_config("c3", V=256, **over)
    _attn_case(cfg, workloads.generate(cfg), split_keys=split)


def test_attention_wide_split_is_deterministic_and_resets_workspace():
    """The second workgroup of a unit merges both halves in chunk order, so
    repeated calls give the same bits whichever finished first; every call
    leaves the workspace's counters at zero."""
    cfg = workloads.get_config("c3", V=256, B=6, L_min=500, L_max=3000)
    inp = workloads.generate(cfg)
    t = oracle_tree(inp, cfg)
    args = [dev(inp[x]) for x in ("q", "k_pool", "v_pool", "page_table", "prefix_len")]
    bits = dev(t["mask_bits"].view(np.int32))
    outs = []
    for _ in range(3):
        out, lse = sdv.sdv_tree_verify_attention(*args, bits, page=cfg.page, want_lse=True)
        torch.cuda.synchronize()
        outs.append((host(out.view(torch.int16)).copy(), host(lse).copy()))
    for i, (o, l) in enumerate(outs[1:], 1):
        do = np.argwhere(o != outs[0][0])
        dl = np.argwhere(l != outs[0][1])
        assert len(do) == 0 and len(dl) == 0, (
            "call %d differs from call 0 at %d outputs / %d lse, (request, node, head) e.g. %s / %s"
            % (i, len(do), len(dl), do[:4].tolist(), dl[:4].tolist()))
    from speculative_decoding_eagle_amd import binding
    key = (torch.cuda.current_device(), torch.cuda.current_stream().cuda_stream)
    ws = binding._ATTN_WS[key]
    assert not host(ws[: 256 + 32768]).any(), "status or counters not reset"


# ------------------------------------------------------------------- A9-A10

def test_tli_maps_and_remaps_bit_exact():
    cfg = workloads.get_config("c5")
    inp = workloads.generate(cfg, with_rows=False)
    say("tli maps")
    gd2t, gt2d = sdv.sdv_tli_build_maps(dev(inp["inter_ids"]), dev(inp["tgt_ids"]), cfg.V_draft, cfg.V,
                                        int(inp["fallback"]))
    torch.cuda.synchronize()
    d2t, t2d = otli.build_maps(inp["inter_ids"], inp["tgt_ids"], cfg.V_draft, cfg.V, int(inp["fallback"]))
    assert np.array_equal(host(gd2t), d2t) and np.array_equal(host(gt2d), t2d)
    rng = workloads.extra_rng(cfg, 5)
    ids_t = np.concatenate([rng.integers(0, cfg.V, 5000), [-1, cfg.V, 2 ** 30]]).astype(np.int32)
    ids_d = np.concatenate([rng.integers(0, cfg.V_draft, 5000), [-5, cfg.V_draft]]).astype(np.int32)
    assert np.array_equal(host(sdv.sdv_tli_map_ids(gt2d, dev(ids_t))), otli.map_ids(t2d, ids_t))
    assert np.array_equal(host(sdv.sdv_tli_map_ids(gd2t, dev(ids_d))), otli.map_ids(d2t, ids_d))


def test_tli_constrain_and_scatter_bit_exact():
    cfg = workloads.get_config("c5")
    inp = workloads.generate(cfg)
    rng = workloads.extra_rng(cfg, 6)
    pruned = rng.standard_normal((cfg.B, cfg.K_inter)).astype(np.float32)
    say("tli constrain")
    full = sdv.sdv_tli_constrain_draft_logits(dev(pruned), dev(inp["inter_ids"]), cfg.V_draft)
    torch.cuda.synchronize()
    assert np.array_equal(host(full), otli.constrain_logits(pruned, inp["inter_ids"], cfg.V_draft))
    say("tli q_scatter")
    q = inp["q_pruned"]
    qt = sdv.sdv_tli_q_scatter(dev(q), dev(inp["tgt_ids"]), cfg.V)
    torch.cuda.synchronize()
    want = otli.q_scatter(q.reshape(-1, cfg.K_inter), inp["tgt_ids"], cfg.V).reshape(cfg.B, cfg.R, cfg.V)
    assert np.array_equal(host(qt), want)


@pytest.mark.parametrize("Vd,Vt,K,rows", [(1001, 999, 300, 5), (1000, 1000, 301, 13), (2048, 4096, 512, 17),
                                          (50000, 60000, 40000, 9), (151936, 128256, 60000, 11),
                                          (151936, 128256, 109568, 3), (1000, 1000, 0, 3)])
def test_tli_constrain_and_scatter_shapes(Vd, Vt, K, rows):
    """Every kernel path: scalar (odd sizes), 16-byte with row groups per XCD
    (K not a multiple of 4), and the LDS gather with one chunk of target ids,
    two, and three, its q rows in one LDS slice, two or three (rows not a multiple
    of the XCD count; the ids on both sides of every chunk and slice boundary
    present); then a second scatter that reuses the inverse left in the
    workspace."""
    rng = np.random.default_rng(Vd + Vt + K)
    inter = np.sort(rng.choice(Vd, K, replace=False)).astype(np.int32)
    tgt = rng.choice(Vt, K, replace=False).astype(np.int32)
    if Vt > 45056:
        edges = [e for c in range(1, (Vt + 45055) // 45056) for e in (45056 * c - 1, 45056 * c)] + [0, Vt - 1]
        rest = np.setdiff1d(tgt, edges)
        tgt = np.concatenate([np.array(edges, np.int32), rng.permutation(rest)[:K - len(edges)]]).astype(np.int32)
        tgt = rng.permutation(tgt).astype(np.int32)
        assert len(np.unique(tgt)) == K
    pruned = rng.standard_normal((rows, K)).astype(np.float32)
    say("tli constrain/scatter shapes", Vd, Vt, K, rows)
    full = sdv.sdv_tli_constrain_draft_logits(dev(pruned), dev(inter), Vd)
    torch.cuda.synchronize()
    assert np.array_equal(host(full), otli.constrain_logits(pruned, inter, Vd))
    # (zero-filled only for K = 0, whose calls leave the workspace untouched;
    # a call that builds the map writes its header itself)
    ws = torch.zeros(sdv._lib.lib().sdv_tli_q_scatter_workspace_size(Vt), dtype=torch.uint8, device="cuda")
    q1 = rng.random((rows, K)).astype(np.float32)
    q2 = rng.random((rows, K)).astype(np.float32)
    g1 = sdv.sdv_tli_q_scatter(dev(q1), dev(tgt), Vt, ws=ws)
    g2 = sdv.sdv_tli_q_scatter(dev(q2), None, Vt, ws=ws)
    torch.cuda.synchronize()
    assert np.array_equal(host(g1), otli.q_scatter(q1, tgt, Vt))
    assert np.array_equal(host(g2), otli.q_scatter(q2, tgt, Vt))
    assert sdv.sdv_workspace_status(ws) == 0
    # a reuse call whose K differs from the map's: zeros and a status bit,
    # never a gather past the row
    if K > 4:
        g3 = sdv.sdv_tli_q_scatter(dev(q2[:, :K - 4].copy()), None, Vt, ws=ws)
        torch.cuda.synchronize()
        assert (host(g3) == 0).all()
        assert sdv.sdv_workspace_status(ws, reset=True) == sdv.STATUS_TLI_REUSE
        assert sdv.sdv_workspace_status(ws) == 0
        g4 = sdv.sdv_tli_q_scatter(dev(q2), None, Vt, ws=ws)          # the reset wiped the map too
        torch.cuda.synchronize()
        assert (host(g4) == 0).all() and sdv.sdv_workspace_status(ws, reset=True) == sdv.STATUS_TLI_REUSE
        g5 = sdv.sdv_tli_q_scatter(dev(q2), dev(tgt), Vt, ws=ws)       # rebuilt
        torch.cuda.synchronize()
        assert np.array_equal(host(g5), otli.q_scatter(q2, tgt, Vt)) and sdv.sdv_workspace_status(ws) == 0


# Up to 64 hidden rows whose 16-row blocks fit in LDS (padded rows, at most
# 160 KB) take the staged kernel (one, two or four blocks: B = 5, 8, 17, 33,
# 48, 64; H = 1248 is the largest that fits at B = 64); more rows (130) or
# wider ones (H = 1280 at B = 64) take the kernel that reads them from L1/L2.
# K = 109569 is the larger intersection of the TLI notes; tails of K below
# a block (77, 241, 500, 4097).
@pytest.mark.parametrize("B,H,K", [(64, 896, 60000), (5, 64, 1000), (17, 96, 77), (130, 32, 513), (33, 896, 4097),
                                   (8, 896, 109569), (64, 1248, 500), (64, 1280, 500), (48, 64, 241)])
def test_tli_lm_head_within_tolerance(B, H, K):
    rng = np.random.default_rng(B + H + K)
    hidden = workloads.to_bf16_bits(rng.standard_normal((B, H)).astype(np.float32))
    w = workloads.to_bf16_bits((rng.standard_normal((K, H)) * 0.02).astype(np.float32))
    say("lm_head", B, H, K)
    g = sdv.sdv_tli_lm_head(dev(hidden), dev(w))
    torch.cuda.synchronize()
    ref = otli.lm_head(hidden, w)
    assert_attention_close(host(g), ref)
    assert np.abs(host(g) - ref).max() < 1e-3


def test_tli_pipeline_c5():
    """Scatter q into the target vocabulary, take its top-1 chain, verify."""
    cfg = workloads.get_config("c5")
    inp = workloads.generate(cfg)
    say("tli pipeline")
    qt = sdv.sdv_tli_q_scatter(dev(inp["q_pruned"]), dev(inp["tgt_ids"]), cfg.V)
    tp, ti = sdv.sdv_draft_topk(qt, 1)
    t = sdv.sdv_build_tree(tp, ti, dev(inp["root_token"]), dev(inp["prefix_len"]), 1, cfg.S, cfg.N)
    r = sdv.sdv_verify_accept(sdv.STOCHASTIC, t, dev(inp["target"]), cfg.S, draft_probs=qt,
                              u_accept=dev(inp["u_accept"]), u_draw=dev(inp["u_draw"]))
    torch.cuda.synchronize()
    q_host = otli.q_scatter(inp["q_pruned"].reshape(-1, cfg.K_inter), inp["tgt_ids"], cfg.V).reshape(cfg.B, cfg.R, cfg.V)
    otp, oti = otopk.draft_topk(q_host, 1)
    ot = otree.build_tree(otp, oti, inp["root_token"], inp["prefix_len"], 1, cfg.S, cfg.N)
    o = oacc.verify_stochastic(ot, inp["target"], q_host, inp["u_accept"], inp["u_draw"], cfg.S)
    for key in o:
        assert np.array_equal(host(r[key]), o[key]), key


# ------------------------------------------------------- degenerate cases

def test_empty_batches_return_without_work():
    """Every stage with an empty batch: success, empty outputs, no launch
    that touches memory."""
    say("empty batches")
    f32, i32 = torch.float32, torch.int32
    e = lambda *s, dt=i32: torch.empty(s, dtype=dt, device="cuda")
    p, i = sdv.sdv_draft_topk(e(0, 100, dt=f32), 4)
    assert p.shape == (0, 4) and i.shape == (0, 4)
    p, i = sdv.sdv_draft_topk_logits(e(0, 100, dt=torch.bfloat16), 4)
    assert p.shape == (0, 4)
    t = sdv.sdv_build_tree(e(0, 9, 2, dt=f32), e(0, 9, 2), e(0), e(0), 2, 5, 8)
    assert t["tokens"].shape == (0, 8)
    c = sdv.sdv_build_chain(e(0, 4, dt=f32), e(0, 4), e(0), e(0))
    assert c["tokens"].shape == (0, 5)
    pool = torch.zeros((64, 2, 64), dtype=torch.bfloat16, device="cuda")
    out, _ = sdv.sdv_tree_verify_attention(e(0, 8, 4, 64, dt=torch.bfloat16), pool, pool, e(0, 16), e(0),
                                           e(0, 8, 1))
    assert out.shape == (0, 8, 4, 64)
    acc = sdv.sdv_verify_accept(sdv.GREEDY, {"tokens": e(0, 8), "next_token": e(0, 8), "next_sibling": e(0, 8),
                                             "q_row": e(0, 8)}, e(0, 8, 100, dt=f32), 5)
    assert acc["accept_len"].shape == (0,)
    new_len, freed, num_freed = sdv.sdv_compact_kv(e(0, 16), e(0), e(0), e(0, 6), 8, 5, 1)
    assert new_len.shape == (0,)
    torch.cuda.synchronize()


@pytest.mark.parametrize("mode", ["greedy", "stochastic"])
def test_single_node_trees_through_every_stage(mode):
    """N = 1: the tree is the root alone; attention sees the prefix and the
    root; the walk commits only the bonus token (argmax, or a draw from p);
    compaction keeps the root and frees nothing."""
    name = "c3" if mode == "greedy" else "c4"
    cfg = workloads.get_config(name, V=300, B=3, N=1, S=1, k=2, L_min=5, L_max=50)
    inp = workloads.generate(cfg)
    t = oracle_tree(inp, cfg)
    say("single node", mode)
    tp, ti = otopk.draft_topk(inp["draft_probs"], cfg.k)
    g = _gpu_tree(tp, ti, inp["root_token"], inp["prefix_len"], cfg.k, cfg.S, cfg.N)
    _assert_tree_equal(g, t)
    _attn_case(cfg, inp)
    if mode == "greedy":
        ga = _gpu_accept(sdv.GREEDY, t, inp["target"], cfg.S)
        o = oacc.verify_greedy(t, inp["target"], cfg.S)
    else:
        ga = _gpu_accept(sdv.STOCHASTIC, t, inp["target"], cfg.S, draft_probs=inp["draft_probs"],
                         u_accept=inp["u_accept"], u_draw=inp["u_draw"])
        o = oacc.verify_stochastic(t, inp["target"], inp["draft_probs"], inp["u_accept"], inp["u_draw"], cfg.S)
    _assert_accept_equal(ga, o)
    assert (o["commit_len"] == 1).all() and (o["accept_len"] == 0).all()
    table = inp["page_table"]
    gt = dev(table)
    pools = ([dev(inp["k_pool"])], [dev(inp["v_pool"])]) if cfg.page > 1 else ([], [])
    new_len, freed, num_freed = sdv.sdv_compact_kv(gt, dev(inp["prefix_len"]), dev(o["accept_len"]),
                                                   dev(o["accept_path"]), cfg.N, cfg.S, cfg.page, *pools)
    torch.cuda.synchronize()
    ot, _, _, onew, ofreed = ocmp.compact_kv(table, [inp["k_pool"]] if cfg.page > 1 else [],
                                             [inp["v_pool"]] if cfg.page > 1 else [], inp["prefix_len"],
                                             o["accept_len"], o["accept_path"], cfg.N, cfg.page)
    assert np.array_equal(host(gt), ot) and np.array_equal(host(new_len), onew)
    assert int(host(num_freed)[0]) == len(ofreed)


# ------------------------------------------------------- device status

def test_status_reports_given_up_waits_and_reset_restores():
    """With the wait limit at 0 every bounded wait between workgroups gives
    up at once (every kernel still exits normally): the top-k piece merge,
    the attention key-split merge and the accept walk's exchanges.  Their
    status bits appear in the workspaces, a reset clears them, and with the
    library's limit the same workspaces give the oracle's results again."""
    rng = np.random.default_rng(4242)
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    rows, V = ncu + 5, 20000                      # rows = CUs + 5: five rows cut into pieces
    p = workloads.softmax_rows(rng.standard_normal((rows, V)).astype(np.float32) * 3)
    cfg = workloads.get_config("c3", B=4)
    inp = workloads.generate(cfg)
    t = oracle_tree(inp, cfg)
    accept_tree = {k: dev(t[k]) for k in ("tokens", "next_token", "next_sibling")}
    bits_dev = dev(t["mask_bits"].view(np.int32))

    def run_all():
        tk = sdv.sdv_draft_topk(dev(p), 8)
        att = sdv.sdv_tree_verify_attention(dev(inp["q"]), dev(inp["k_pool"]), dev(inp["v_pool"]),
                                            dev(inp["page_table"]), dev(inp["prefix_len"]),
                                            bits_dev, page=cfg.page)[0]
        acc = sdv.sdv_verify_accept(sdv.GREEDY, accept_tree, dev(inp["target"]), cfg.S)
        torch.cuda.synchronize()
        return tk, att, acc

    sdv.device_status(reset=True)
    say("status: wait limit 0")
    prev = sdv.sdv_set_wait_limit(0)
    try:
        run_all()
    finally:
        sdv.sdv_set_wait_limit(prev)
    bits = sdv.device_status(reset=False)
    assert bits & sdv.STATUS_TOPK_MERGE_WAIT
    assert bits & sdv.STATUS_ATTN_MERGE_WAIT
    assert bits & sdv.STATUS_ACCEPT_WAIT
    assert sdv.device_status(reset=True) == bits
    assert sdv.device_status(reset=False) == 0
    say("status: library limit, after the reset")
    (gp, gi), att, acc = run_all()
    assert sdv.device_status(reset=False) == 0
    op, oi = otopk.draft_topk(p, 8)
    assert np.array_equal(host(gi), oi) and np.array_equal(host(gp), op)
    ref, _ = oatt.tree_verify_attention(inp["q"], inp["k_pool"], inp["v_pool"], inp["page_table"],
                                        inp["prefix_len"], t["mask"], cfg.page)
    assert_attention_close(bf16_to_f64(att), ref)
    want = oacc.verify_greedy(t, inp["target"], S=cfg.S)
    for key in want:
        assert np.array_equal(host(acc[key]), want[key]), key


# ------------------------------------- sampling primitives, device vs host

def test_sampling_primitives_at_their_edges_device_vs_host():
    """The stochastic walk on requests built to sit on the contract's edges
    (tests/_sampling_edges.py): equality in the accept test, normalised
    residuals whose fp64 quotient is an fp32 midpoint or one fp64 ulp off
    one, S near 2^56 that fp64 cannot hold, draws whose threshold meets a
    running mass exactly at a vocabulary-slice boundary, masses below 2^-40,
    kk = 0 and 2^24 - 1, S below 2^24 and near 2^57.  The kernel's u64 -> f64
    conversion, fp64 divide, fp32 rounding, floor(w * 2^40) and inverse-CDF
    threshold must reproduce the oracle's bit for bit."""
    import _sampling_edges as edges
    inp, cases = edges.build()
    tree = {k: dev(inp[k]) for k in ("tokens", "next_token", "next_sibling", "q_row")}
    say("sampling edges", len(cases), "requests")
    g = sdv.sdv_verify_accept(sdv.STOCHASTIC, tree, dev(inp["target"]), 1, draft_probs=dev(inp["draft_probs"]),
                              u_accept=dev(inp["u_accept"]), u_draw=dev(inp["u_draw"]))
    torch.cuda.synchronize()
    want = oacc.verify_stochastic({k: inp[k] for k in ("tokens", "next_token", "next_sibling", "q_row")},
                                  inp["target"], inp["draft_probs"], inp["u_accept"], inp["u_draw"], S=1)
    assert sdv.device_status(reset=True) == 0
    for key in want:
        got = host(g[key])
        bad = [cases[b]["name"] for b in range(len(cases)) if not np.array_equal(got[b], want[key][b])]
        assert not bad, "%s differs for %s" % (key, bad)
