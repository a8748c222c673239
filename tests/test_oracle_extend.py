"""Pins of the oracle's draft-extend index preparation: the pages' row
alignment (row i predicts token i+1) and worked example, the tree structure
the accept walk moved through, TLI's target -> draft -> target round trip, and
the degenerate batches."""
import json
import os

import numpy as np
import pytest

from oracle import accept as oacc
from oracle import extend as oext
from oracle import tli as otli
import workloads
from _helpers import oracle_tree, plant_greedy
from test_oracle_accept import chain_tree, onehot_rows


def _golden(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


def test_extend_row_alignment(golden_dir):
    """Prefix 5, draft 3, everything accepted: rows 4..7 chose the four
    committed tokens, and row i predicts token i+1, so the extend's tokens sit
    at positions 5..8 and pair with the hidden states of rows 4..7."""
    g = _golden(golden_dir, "row_alignment.json")
    L, k = g["prefix_len"], g["draft_len"]
    rows = g["verify_rows"] + [g["bonus_row"]]
    props = [20 + r for r in g["verify_rows"]]
    t = chain_tree(3, props, prefix_len=L - 1)
    r = oacc.verify_greedy(t, onehot_rows([20 + x for x in range(L + k)], 64)[t["positions"][0]][None], S=k)
    e = oext.draft_extend_prep(np.array([L - 1]), r["commit_len"], r["commit_tokens"], r["accept_path"], N=k + 1)
    assert e["positions"].tolist() == [x + 1 for x in rows]
    assert t["positions"][0][e["hidden_index"]].tolist() == rows
    assert e["input_ids"].tolist() == props + [20 + g["bonus_row"]]
    assert e["extend_start"].tolist() == [0, k + 1]
    assert e["last_index"].tolist() == [k]
    assert e["seq_len"].tolist() == [L + k + 1]


def test_extend_worked_example(golden_dir):
    """Draft [1,1,1], target 1 then 2: the extend runs over [1, 2], chosen at
    the root and at the first draft node."""
    g = _golden(golden_dir, "greedy_worked_example.json")
    props = g["proposals"]
    L = 7
    t = chain_tree(0, props, prefix_len=L)
    choices = g["target_choices"] + [5] * (len(props) + 1 - len(g["target_choices"]))
    r = oacc.verify_greedy(t, onehot_rows(choices, 8)[None], S=len(props))
    e = oext.draft_extend_prep(np.array([L]), r["commit_len"], r["commit_tokens"], r["accept_path"],
                               N=len(props) + 1)
    assert e["input_ids"].tolist() == g["expected_commit"]
    assert e["positions"].tolist() == [L + 1, L + 2]
    assert e["hidden_index"].tolist() == [0, 1]
    assert e["last_index"].tolist() == [1] and e["seq_len"].tolist() == [L + 3]


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_extend_follows_the_accepted_path(seed):
    """On seeded trees with planted acceptance: the rows of a request are
    contiguous and in commit order; the node that chose committed token j has
    depth j (so its position + 1 is the token's position); and every
    committed token but a correction or bonus is the token of the next node
    on the path."""
    cfg = workloads.get_config("c3", V=300, B=12)
    inp = workloads.generate(cfg, with_attention=False)
    t = oracle_tree(inp, cfg)
    rng = np.random.default_rng(seed)
    target = plant_greedy(inp["target"], t, rng, cfg.S)
    rem = rng.integers(0, cfg.S + 2, size=cfg.B).astype(np.int32)
    r = oacc.verify_greedy(t, target, S=cfg.S, remaining=rem)
    e = oext.draft_extend_prep(inp["prefix_len"], r["commit_len"], r["commit_tokens"], r["accept_path"], N=cfg.N)
    st = e["extend_start"]
    assert st[0] == 0 and np.array_equal(np.diff(st), r["commit_len"])
    assert (r["commit_len"] == 0).any() and (r["commit_len"] > 2).any()      # both kinds occur
    for b in range(cfg.B):
        c = int(r["commit_len"][b])
        L = int(inp["prefix_len"][b])
        for j in range(c):
            row = st[b] + j
            node = e["hidden_index"][row] - b * cfg.N
            assert 0 <= node < cfg.N
            assert t["depth"][b, node] == j
            assert e["positions"][row] == t["positions"][b, node] + 1 == L + 1 + j
            assert e["input_ids"][row] == r["commit_tokens"][b, j]
            if j + 1 <= r["accept_len"][b]:
                assert e["input_ids"][row] == t["tokens"][b, r["accept_path"][b, j + 1]]
        assert e["last_index"][b] == (st[b] + c - 1 if c else -1)
        assert e["seq_len"][b] == L + 1 + c


def test_extend_tli_round_trip():
    """Under TLI the extend reads draft ids; mapping them back gives the
    committed target ids wherever the target id is in the intersection, and
    the fallback's image elsewhere."""
    rng = np.random.default_rng(5)
    Vd, Vt, K = 500, 400, 120
    inter = np.sort(rng.choice(Vd, K, replace=False)).astype(np.int32)
    tgt = rng.choice(Vt, K, replace=False).astype(np.int32)
    fallback = int(np.setdiff1d(np.arange(Vd), inter)[0])
    d2t, t2d = otli.build_maps(inter, tgt, Vd, Vt, fallback)
    B, S = 6, 4
    commit_len = np.array([5, 0, 3, 1, 5, 2], np.int32)
    commit = np.full((B, S + 1), -1, np.int32)
    path = np.full((B, S + 1), -1, np.int32)
    for b in range(B):
        c = commit_len[b]
        commit[b, :c] = np.where(rng.random(c) < 0.7, rng.choice(tgt, c), rng.integers(0, Vt, c))
        path[b, :max(c, 1)] = np.arange(max(c, 1))
    e = oext.draft_extend_prep(np.arange(B) * 10, commit_len, commit, path, N=8, t2d=t2d)
    flat = np.concatenate([commit[b, :commit_len[b]] for b in range(B)])
    inside = np.isin(flat, tgt)
    assert np.array_equal(d2t[e["input_ids"][inside]], flat[inside])
    assert (e["input_ids"][~inside] == fallback).all() and (~inside).any()
    plain = oext.draft_extend_prep(np.arange(B) * 10, commit_len, commit, path, N=8)
    assert np.array_equal(plain["input_ids"], flat)
    for key in ("positions", "hidden_index", "extend_start", "last_index", "seq_len"):
        assert np.array_equal(plain[key], e[key])


def test_extend_degenerate_and_rejects():
    e = oext.draft_extend_prep(np.zeros(0, np.int32), np.zeros(0, np.int32), np.zeros((0, 3), np.int32),
                               np.zeros((0, 3), np.int32), N=4)
    assert e["extend_start"].tolist() == [0] and e["input_ids"].size == 0
    e = oext.draft_extend_prep(np.array([3, 9]), np.array([0, 0]), np.full((2, 3), -1), np.full((2, 3), -1), N=4)
    assert e["last_index"].tolist() == [-1, -1] and e["seq_len"].tolist() == [4, 10]
    with pytest.raises(ValueError):
        oext.draft_extend_prep(np.array([0]), np.array([4]), np.zeros((1, 3), np.int32), np.zeros((1, 3), np.int32), N=4)
    with pytest.raises(ValueError):
        oext.draft_extend_prep(np.array([0]), np.array([2]), np.array([[1, -1, -1]]), np.array([[0, 1, -1]]), N=4)
