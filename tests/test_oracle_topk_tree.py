"""Pins of the oracle's draft top-k and tree build against facts outside it."""
import functools
import json
import os

import numpy as np
import pytest

from oracle import topk as otopk
from oracle import tree as otree
import workloads


# ------------------------------------------------------------------ top-k

def test_topk_k1_is_library_argmax():
    rng = np.random.default_rng(1)
    p = rng.random((50, 333)).astype(np.float32)
    p[7, 10] = p[7, 200] = 2.0                     # a tie: the lower id wins
    vals, ids = otopk.draft_topk(p, 1)
    assert np.array_equal(ids[:, 0], np.argmax(p, axis=1))
    assert ids[7, 0] == 10
    assert np.array_equal(vals[:, 0], p.max(axis=1))


def test_topk_matches_python_sorted_with_ties():
    rng = np.random.default_rng(2)
    # few distinct values -> many ties
    p = (rng.integers(0, 6, size=(40, 57)) / 8.0).astype(np.float32)
    for k in (1, 2, 5, 8, 57):
        vals, ids = otopk.draft_topk(p, k)
        for r in range(p.shape[0]):
            want = sorted(range(p.shape[1]), key=lambda i: (-float(p[r, i]), i))[:k]
            assert ids[r].tolist() == want
            assert vals[r].tolist() == [float(p[r, i]) for i in want]


def test_topk_rejects_bad_k():
    with pytest.raises(ValueError):
        otopk.draft_topk(np.zeros((1, 4), np.float32), 5)


# ------------------------------------------- fused softmax + top-k (logits)

import math


def test_fused_two_entries_follow_the_logistic_function():
    """softmax of two logits is the logistic function of their difference."""
    for a, b, T in [(1.5, -0.25, 1.0), (0.0, 3.0, 0.7), (-2.0, -2.5, 1.3), (10.0, -10.0, 2.0)]:
        vals, ids = otopk.draft_topk_from_logits(np.array([[a, b]], np.float32), 2, T)
        hi, lo = (a, b) if a >= b else (b, a)
        p_hi = 1.0 / (1.0 + math.exp(-(hi - lo) / T))
        assert ids[0].tolist() == ([0, 1] if a >= b else [1, 0])
        assert abs(vals[0, 0] - p_hi) < 1e-15 and abs(vals[0, 1] - (1.0 - p_hi)) < 1e-15


def test_fused_is_invariant_to_shift_and_to_scaling_logits_with_the_temperature():
    rng = np.random.default_rng(7)
    x = (rng.standard_normal((6, 300)) * 3.0).astype(np.float32)
    v0, i0 = otopk.draft_topk_from_logits(x, 8, 0.8)
    v1, i1 = otopk.draft_topk_from_logits(x + np.float32(5.0), 8, 0.8)    # the shift rounds in fp32: 1e-5
    v2, i2 = otopk.draft_topk_from_logits(x * np.float32(2.0), 8, 1.6)    # x*2 is exact in fp32
    assert np.array_equal(i0, i1) and np.array_equal(i0, i2)
    assert np.allclose(v0, v1, rtol=1e-5, atol=0) and np.allclose(v0, v2, rtol=1e-13, atol=0)


def test_fused_uniform_row_gives_lowest_ids_and_one_over_V():
    vals, ids = otopk.draft_topk_from_logits(np.full((2, 40), 0.5, np.float32), 5, 1.0)
    assert ids.tolist() == [[0, 1, 2, 3, 4]] * 2
    assert np.allclose(vals, 1.0 / 40, rtol=1e-15, atol=0)


def test_fused_excluded_entries_get_zero_and_the_rest_renormalise():
    x = np.full((1, 10), -np.inf, np.float32)
    x[0, [2, 5, 7]] = [1.0, 3.0, 1.0]
    vals, ids = otopk.draft_topk_from_logits(x, 5, 1.0)
    z = math.exp(1.0) * 2 + math.exp(3.0)
    assert ids[0].tolist() == [5, 2, 7, 0, 1]
    assert np.allclose(vals[0, :3], [math.exp(3.0) / z, math.exp(1.0) / z, math.exp(1.0) / z], rtol=1e-15)
    assert vals[0, 3] == 0.0 and vals[0, 4] == 0.0


def test_fused_agrees_with_processed_rows_and_the_plain_top_k():
    """The generator's softmax (an independent float64 evaluation, rounded
    once to fp32) followed by the plain top-k gives the same ids where the
    rounded probabilities do not tie, and values within that rounding."""
    rng = np.random.default_rng(11)
    x = (rng.standard_normal((12, 4099)) * 3.0).astype(np.float32)
    for T in (1.0, 0.7):
        pv, pi = otopk.draft_topk_from_logits(x, 8, T)
        rows = workloads.softmax_rows(x, T)
        qv, qi = otopk.draft_topk(rows, 9)
        for r in range(x.shape[0]):
            if len(set(qv[r].tolist())) == 9:
                assert pi[r].tolist() == qi[r, :8].tolist()
        assert np.all(np.abs(pv - qv[:, :8].astype(np.float64)) <= 2.0 ** -24 * pv)


def test_fused_orders_by_exact_probability_not_by_rounded_values():
    """Logits 0 and 2^-30 give fp32 probabilities that round alike, so the
    plain top-k of the rounded row puts the lower id first; the exact
    probabilities order the larger logit first."""
    x = np.full((1, 5000), -30.0, np.float32)
    x[0, 3] = 0.0
    x[0, 9] = np.float32(2.0 ** -30)
    rows = workloads.softmax_rows(x, 1.0)
    assert rows[0, 3] == rows[0, 9] and otopk.draft_topk(rows, 2)[1][0].tolist() == [3, 9]
    vals, ids = otopk.draft_topk_from_logits(x, 2, 1.0)
    assert ids[0].tolist() == [9, 3]
    assert vals[0, 0] > vals[0, 1]


def test_fused_reads_bf16_bit_patterns():
    bits = np.array([[0x3F80, 0x4000, 0xFF80, 0xBF80]], np.uint16)    # 1, 2, -inf, -1
    vb, ib = otopk.draft_topk_from_logits(bits, 4, 1.0, bf16=True)
    vf, iff = otopk.draft_topk_from_logits(np.array([[1.0, 2.0, -np.inf, -1.0]], np.float32), 4, 1.0)
    assert ib.tolist() == [[1, 0, 3, 2]] and np.array_equal(ib, iff) and np.array_equal(vb, vf)


def test_fused_full_row_sums_to_one():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((3, 257)) * 4.0).astype(np.float32)
    vals, ids = otopk.draft_topk_from_logits(x, 257, 1.1)
    assert np.allclose(vals.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    for r in range(3):
        assert ids[r].tolist() == sorted(range(257), key=lambda i: (-float(x[r, i]), i))


def test_fused_rejects_bad_input():
    with pytest.raises(ValueError):
        otopk.draft_topk_from_logits(np.zeros((1, 4), np.float32), 2, 0.0)
    with pytest.raises(ValueError):
        otopk.draft_topk_from_logits(np.array([[0.0, np.nan]], np.float32), 1, 1.0)
    with pytest.raises(ValueError):
        otopk.draft_topk_from_logits(np.full((1, 3), -np.inf, np.float32), 1, 1.0)
    with pytest.raises(ValueError):
        otopk.draft_topk_from_logits(np.zeros((1, 4), np.float32), 5, 1.0)


# ------------------------------------------------------------------- tree

def _golden(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


@pytest.mark.parametrize("N", [6, 7])
def test_tree_hand_worked_example(golden_dir, N):
    g = _golden(golden_dir, "hand_tree_k2s3.json")
    tp = np.array([g["topk_p"]], np.float32)
    ti = np.array([g["topk_id"]], np.int32)
    t = otree.build_tree(tp, ti, np.array([g["root_token"]]), np.array([g["prefix_len"]]),
                         g["k"], g["S"], N)
    want = g["N%d" % N]
    for key in ("tokens", "parent", "depth", "q_row", "next_token", "next_sibling"):
        assert t[key][0].tolist() == want[key], key
    assert t["score"][0].tolist() == want["score"]
    if "positions" in want:
        assert t["positions"][0].tolist() == want["positions"]
    if "mask_rows" in want:
        for i, row in enumerate(want["mask_rows"]):
            assert np.flatnonzero(t["mask"][0, i]).tolist() == row
    assert t["retrieve_index"][0].tolist() == list(range(N))


def test_exercise_frontier_count(golden_dir):
    """num_steps=3, topk=4: the steps expand 4+4+4 = 12 frontier candidates."""
    g = _golden(golden_dir, "exercise_candidates.json")
    k, S = g["topk"], g["num_steps"]
    rng = np.random.default_rng(3)
    probs = workloads.softmax_rows(rng.standard_normal((1, 1 + (S - 1) * k, 64)).astype(np.float32))
    tp, ti = otopk.draft_topk(probs, k)
    tb = otree.TreeBuilder(k, S)
    tb.start(tp[0, 0], ti[0, 0])
    frontiers = [list(tb.frontier)]
    for _ in range(1, S):
        rows = tb.frontier_rows()
        tb.expand([tp[0, r] for r in rows], [ti[0, r] for r in rows])
        frontiers.append(list(tb.frontier))
    assert sum(len(f) for f in frontiers) == g["expanded_candidates"]
    # draft passes: one per step plus the draft extend; the verify is one target pass
    assert S + 1 == g["draft_passes"]
    # the root's row and one row per frontier slot of every step but the last
    assert workloads.num_draft_rows(k, S) == 1 + (S - 1) * k


def test_k1_is_a_chain():
    """topk=1: the tree is the chain of top-1 tokens, N = S + 1."""
    rng = np.random.default_rng(4)
    S = 5
    probs = workloads.softmax_rows(rng.standard_normal((3, S, 100)).astype(np.float32))
    tp, ti = otopk.draft_topk(probs, 1)
    t = otree.build_tree(tp, ti, np.array([1, 2, 3]), np.array([10, 20, 30]), 1, S, S + 1)
    for b in range(3):
        assert t["parent"][b].tolist() == [-1] + list(range(S))
        assert t["tokens"][b, 1:].tolist() == [int(np.argmax(probs[b, r])) for r in range(S)]
        assert t["depth"][b].tolist() == list(range(S + 1))
        assert t["positions"][b].tolist() == [10 * (b + 1) + d for d in range(S + 1)]
        assert t["q_row"][b].tolist() == list(range(S)) + [-1]


def _chain_inputs(seed, B=3, S=6, V=120):
    rng = np.random.default_rng(seed)
    probs = workloads.softmax_rows(rng.standard_normal((B, S, V)).astype(np.float32))
    tp, ti = otopk.draft_topk(probs, 1)
    root = rng.integers(0, V, size=B).astype(np.int32)
    prefix = rng.integers(0, 500, size=B).astype(np.int32)
    return probs, tp, ti, root, prefix


def test_multilayer_chain_follows_the_step_slicing():
    """Multi-layer draft (per-step layers, per-step top-1 concatenated): node
    i+1 is step i's token, its parent is node i (the root for step 0), and it
    keeps its own step's probability as its score; the mask is the lower
    triangle and every node has one child."""
    probs, tp, ti, root, prefix = _chain_inputs(7)
    B, S = tp.shape[:2]
    N = S + 1
    c = otree.build_chain(tp[:, :, 0], ti[:, :, 0], root, prefix)
    for b in range(B):
        assert c["parent"][b].tolist() == [-1] + list(range(S))
        assert c["tokens"][b].tolist() == [int(root[b])] + [int(np.argmax(probs[b, i])) for i in range(S)]
        assert c["score"][b, 0] == 1.0 and np.array_equal(c["score"][b, 1:], tp[b, :, 0])
        assert np.array_equal(c["mask"][b], np.tril(np.ones((N, N), np.uint8)))
        assert c["next_token"][b].tolist() == list(range(1, N)) + [-1]
        assert (c["next_sibling"][b] == -1).all()
        assert c["positions"][b].tolist() == [int(prefix[b]) + d for d in range(N)]
        assert c["retrieve_index"][b].tolist() == [b * N + i for i in range(N)]


@pytest.mark.parametrize("seed,S", [(8, 1), (9, 5), (10, 12)])
def test_multilayer_chain_is_the_k1_tree_with_step_scores(seed, S):
    """The same per-step lists read in the tree layout [B, R=S, k=1] build
    the same tree; the tree's scores are the running fp32 products of the
    chain's step scores, root first."""
    probs, tp, ti, root, prefix = _chain_inputs(seed, S=S)
    c = otree.build_chain(tp, ti, root, prefix)
    t = otree.build_tree(tp, ti, root, prefix, 1, S, S + 1)
    for key in t:
        if key != "score":
            assert np.array_equal(c[key], t[key]), key
    for b in range(tp.shape[0]):
        run = [np.float32(1.0)]
        for x in c["score"][b, 1:]:
            run.append(np.float32(run[-1] * x))
        assert np.array_equal(np.array(run, np.float32), t["score"][b])


def test_multilayer_chain_rejects_wider_lists():
    _, tp, ti, root, prefix = _chain_inputs(11)
    with pytest.raises(ValueError):
        otree.build_chain(np.repeat(tp, 2, axis=2), np.repeat(ti, 2, axis=2), root, prefix)


def _brute_tree(tp, ti, k, S, N):
    """Independent restatement on paths: a candidate carries the list of draft
    probabilities along its path from the root; its score is the left fold of
    fp32 products over that list; its pool key is (step, parent's frontier
    slot, child rank)."""
    def score(cand):
        return functools.reduce(lambda a, x: np.float32(a * np.float32(x)), cand[1], np.float32(1.0))

    cands = []   # (key, path probabilities, token, parent key)
    level = [((0, 0, c), [tp[0][c]], int(ti[0][c]), None) for c in range(k)]
    cands.extend(level)
    for i in range(1, S):
        ranked = sorted(level, key=lambda e: (-float(score(e)), e[0]))[:k]
        nxt = []
        for j, par in enumerate(ranked):
            row = 1 + (i - 1) * k + j
            for c in range(k):
                nxt.append(((i, j, c), par[1] + [tp[row][c]], int(ti[row][c]), par[0]))
        cands.extend(nxt)
        level = nxt
    chosen = sorted(cands, key=lambda e: (-float(score(e)), e[0]))[:N - 1]
    chosen.sort(key=lambda e: e[0])
    return [(c[0], score(c), c[2], c[3]) for c in chosen]


@pytest.mark.parametrize("k,S,N,seed", [(2, 3, 6, 0), (2, 3, 11, 1), (3, 3, 9, 2), (4, 4, 32, 3),
                                        (8, 3, 40, 4), (2, 5, 19, 5), (3, 2, 13, 6)])
def test_tree_matches_brute_force_on_paths(k, S, N, seed):
    rng = np.random.default_rng(seed)
    R = 1 + (S - 1) * k
    # coarse probabilities -> frequent score ties
    probs = (rng.integers(1, 9, size=(1, R, 24)) / 16.0).astype(np.float32)
    tp, ti = otopk.draft_topk(probs, k)
    t = otree.build_tree(tp, ti, np.array([5]), np.array([0]), k, S, N)
    chosen = _brute_tree(tp[0], ti[0], k, S, N)
    assert t["tokens"][0, 1:].tolist() == [c[2] for c in chosen]
    assert t["score"][0, 1:].tolist() == [float(c[1]) for c in chosen]
    assert t["depth"][0, 1:].tolist() == [c[0][0] + 1 for c in chosen]
    key_to_node = {c[0]: i + 1 for i, c in enumerate(chosen)}
    assert t["parent"][0, 1:].tolist() == [0 if c[3] is None else key_to_node[c[3]] for c in chosen]


def test_tree_invariants_on_config_shapes():
    """Ancestor closure, depth, mask = reflexive-transitive closure of parent,
    retrieve lists = children in ascending order, scores = path products."""
    for name in ("c1", "c3", "c4"):
        cfg = workloads.get_config(name, V=512, B=3)
        inp = workloads.generate(cfg, with_attention=False)
        tp, ti = otopk.draft_topk(inp["draft_probs"], cfg.k)
        t = otree.build_tree(tp, ti, inp["root_token"], inp["prefix_len"], cfg.k, cfg.S, cfg.N)
        for b in range(cfg.B):
            par = t["parent"][b]
            for i in range(1, cfg.N):
                assert 0 <= par[i] < i
                assert t["depth"][b, i] == t["depth"][b, par[i]] + 1
                # the node's token is one of its parent's draft row's top-k, and
                # its score is parent score x that probability (fp32)
                r = t["q_row"][b, par[i]]
                c = ti[b, r].tolist().index(t["tokens"][b, i])
                assert t["score"][b, i] == np.float32(t["score"][b, par[i]] * tp[b, r, c])
                anc = set()
                j = i
                while j >= 0:
                    anc.add(j)
                    j = par[j]
                assert set(np.flatnonzero(t["mask"][b, i]).tolist()) == anc
                assert t["mask"][b, i].sum() == t["depth"][b, i] + 1
                for j in range(cfg.N):
                    bit = (int(t["mask_bits"][b, i, j // 32]) >> (j % 32)) & 1
                    assert bit == t["mask"][b, i, j]
            for u in range(cfg.N):
                kids = [i for i in range(1, cfg.N) if par[i] == u]
                walk, c = [], t["next_token"][b, u]
                while c >= 0:
                    walk.append(int(c))
                    c = t["next_sibling"][b, c]
                assert walk == kids
                if kids:
                    assert t["q_row"][b, u] >= 0
            assert t["depth"][b].max() <= cfg.S


def test_full_pool_tree_structure():
    """N - 1 = M: the tree is every expansion; k=2, S=2 -> a full binary tree."""
    rng = np.random.default_rng(9)
    probs = workloads.softmax_rows(rng.standard_normal((1, 3, 50)).astype(np.float32))
    tp, ti = otopk.draft_topk(probs, 2)
    t = otree.build_tree(tp, ti, np.array([0]), np.array([0]), 2, 2, 7)
    assert t["parent"][0].tolist() == [-1, 0, 0, 1, 1, 2, 2]
    assert sorted(t["depth"][0].tolist()) == [0, 1, 1, 2, 2, 2, 2]
