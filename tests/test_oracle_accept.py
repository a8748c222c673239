"""Pins of the oracle's accept walk: the pages' worked examples, exact
enumeration of the rejection sampler, and target-only equivalence of greedy
speculative decoding on tiny deterministic models."""
import json
import os
import zlib
from fractions import Fraction

import numpy as np
import pytest

from oracle import accept as oacc
from oracle import topk as otopk
from oracle import tree as otree
import workloads


def _golden(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


def chain_tree(root, proposals, prefix_len=0):
    n = len(proposals) + 1
    tokens = np.array([root] + list(proposals), np.int32)
    parent = np.arange(-1, n - 1, dtype=np.int32)
    depth = np.arange(n, dtype=np.int32)
    t = otree.verify_arrays(tokens, parent, depth, np.ones(n, np.float32),
                            np.array(list(range(n - 1)) + [-1], np.int32), prefix_len, 0)
    return {k: v[None] for k, v in t.items()}


def onehot_rows(choices, V):
    rows = np.zeros((len(choices), V), np.float32)
    for i, c in enumerate(choices):
        rows[i, c] = 1.0
    return rows


# ------------------------------------------------------------ greedy pins

def test_greedy_worked_example(golden_dir):
    g = _golden(golden_dir, "greedy_worked_example.json")
    props = g["proposals"]
    t = chain_tree(0, props)
    # rows beyond the first mismatch hold arbitrary choices; they must not matter
    choices = g["target_choices"] + [5] * (len(props) + 1 - len(g["target_choices"]))
    for filler in (5, 1):
        choices[2:] = [filler] * (len(choices) - 2)
        r = oacc.verify_greedy(t, onehot_rows(choices, 8)[None], S=len(props))
        n = r["commit_len"][0]
        assert r["commit_tokens"][0, :n].tolist() == g["expected_commit"]
        assert r["accept_len"][0] == g["expected_accept_len"]
        assert r["next_root"][0] == g["expected_commit"][-1]
        assert r["accept_path"][0].tolist() == [0, 1, -1, -1]


def test_row_alignment_quiz(golden_dir):
    """Prefix 5, draft 3: rows 4, 5, 6 verify, row 7 picks the bonus."""
    g = _golden(golden_dir, "row_alignment.json")
    L, k = g["prefix_len"], g["draft_len"]
    V = 64
    full_rows = onehot_rows([20 + r for r in range(L + k)], V)     # row r chooses 20 + r
    props = [20 + r for r in g["verify_rows"]]                     # every draft accepted
    # the root is the last committed token, so the cached prefix is L - 1 tokens
    t = chain_tree(3, props, prefix_len=L - 1)
    assert t["positions"][0].tolist() == g["verify_rows"] + [g["bonus_row"]]
    target = full_rows[t["positions"][0]][None]
    r = oacc.verify_greedy(t, target, S=k)
    assert r["accept_len"][0] == k
    assert r["commit_tokens"][0].tolist() == props + [20 + g["bonus_row"]]


def test_greedy_on_hand_tree(golden_dir):
    g = _golden(golden_dir, "hand_tree_k2s3.json")
    t = otree.build_tree(np.array([g["topk_p"]], np.float32), np.array([g["topk_id"]], np.int32),
                         np.array([g["root_token"]]), np.array([g["prefix_len"]]), 2, 3, 6)
    target = onehot_rows(g["greedy"]["argmax_per_node"], 128)[None]
    r = oacc.verify_greedy(t, target, S=3)
    a = r["accept_len"][0]
    assert r["accept_path"][0, :a + 1].tolist() == g["greedy"]["expected_accept_path"]
    assert r["commit_tokens"][0, :r["commit_len"][0]].tolist() == g["greedy"]["expected_commit"]


def test_budget_and_eos():
    t = chain_tree(0, [1, 2, 3])
    target = onehot_rows([1, 2, 3, 4], 8)[None]
    r = oacc.verify_greedy(t, target, S=3, remaining=np.array([0]))
    assert r["commit_len"][0] == 0 and r["accept_len"][0] == 0 and r["next_root"][0] == -1
    r = oacc.verify_greedy(t, target, S=3, remaining=np.array([2]))
    assert r["commit_tokens"][0, :2].tolist() == [1, 2] and r["commit_len"][0] == 2
    assert r["accept_len"][0] == 2          # both matched drafts keep their KV
    r = oacc.verify_greedy(t, target, S=3, eos_id=2)
    assert r["commit_tokens"][0, :2].tolist() == [1, 2] and r["commit_len"][0] == 2
    r = oacc.verify_greedy(t, target, S=3)
    assert r["commit_tokens"][0].tolist() == [1, 2, 3, 4] and r["accept_len"][0] == 3


# --------------------------------------------- target-only equivalence

class TinyLM:
    """Deterministic float64 next-token logits of a prefix: random embeddings
    mixed over a short window, optionally plus prefix-seeded noise."""

    def __init__(self, V, seed, noise=0.0, noise_seed=0, window=3, d=16):
        rng = np.random.default_rng(seed)
        self.E = rng.standard_normal((V, d))
        self.W = rng.standard_normal((d, V)) * 1.5
        self.V, self.noise, self.noise_seed, self.window = V, noise, noise_seed, window

    def logits(self, seq):
        h = np.zeros(self.E.shape[1])
        for w, tok in enumerate(reversed(seq[-self.window:])):
            h += (0.6 ** w) * self.E[tok]
        out = np.tanh(h) @ self.W
        if self.noise:
            key = zlib.crc32(np.asarray(seq, np.int64).tobytes()) ^ self.noise_seed
            out = out + self.noise * np.random.default_rng(key).standard_normal(self.V)
        return out

    def probs(self, seq):
        z = self.logits(seq)
        e = np.exp(z - z.max())
        return (e / e.sum()).astype(np.float32)


def speculative_round(target, draft, seq, k, S, N, remaining=None, eos_id=-1):
    tb = otree.TreeBuilder(k, S)
    p0, i0 = otopk.draft_topk(draft.probs(seq)[None], k)
    tb.start(p0[0], i0[0])
    for _ in range(1, S):
        rows_p, rows_i = [], []
        for e in tb.frontier:
            p, i = otopk.draft_topk(draft.probs(seq + tb.path_tokens(e))[None], k)
            rows_p.append(p[0])
            rows_i.append(i[0])
        tb.expand(rows_p, rows_i)
    t = tb.finalize(N, seq[-1], len(seq) - 1)
    rows = []
    for u in range(N):
        path, v = [], u
        while v > 0:
            path.append(int(t["tokens"][v]))
            v = int(t["parent"][v])
        rows.append(target.logits(seq + path[::-1]))
    tree = {key: val[None] for key, val in t.items()}
    rem = None if remaining is None else np.array([remaining])
    r = oacc.verify_greedy(tree, np.array(rows)[None], S=S, eos_id=eos_id, remaining=rem)
    return r["commit_tokens"][0, :r["commit_len"][0]].tolist(), int(r["accept_len"][0])


@pytest.mark.parametrize("k,S,N,V,noise", [(1, 4, 5, 16, 0.3), (2, 3, 6, 32, 0.5),
                                           (4, 3, 10, 48, 0.8), (3, 4, 12, 64, 0.2),
                                           (8, 2, 9, 24, 1.0)])
def test_greedy_speculation_equals_target_only(k, S, N, V, noise):
    target = TinyLM(V, seed=V + k)
    draft = TinyLM(V, seed=V + k, noise=noise, noise_seed=7)
    prompt = [1, 2, 3]
    budget = 40
    ref = list(prompt)
    while len(ref) < len(prompt) + budget:
        ref.append(int(np.argmax(target.logits(ref))))
    seq = list(prompt)
    accepted = 0
    while len(seq) < len(prompt) + budget:
        out, a = speculative_round(target, draft, seq, k, S, N,
                                   remaining=len(prompt) + budget - len(seq))
        assert 1 <= len(out) <= S + 1
        seq += out
        accepted += a
    assert seq == ref
    assert accepted > 0          # the draft is good enough to be accepted sometimes


def test_greedy_speculation_with_eos_stops_like_target_only():
    V = 20
    target = TinyLM(V, seed=3)
    draft = TinyLM(V, seed=3, noise=0.3, noise_seed=1)
    ref = [4]
    while True:
        ref.append(int(np.argmax(target.logits(ref))))
        if len(ref) > 60:
            break
    eos = ref[10]                 # some token the target emits
    stop = ref.index(eos, 1)
    seq = [4]
    while seq[-1] != eos or len(seq) == 1:
        out, _ = speculative_round(target, draft, seq, 2, 3, 6, eos_id=eos)
        seq += out
        if eos in out:
            assert out[-1] == eos
            break
    assert seq == ref[:stop + 1]


# --------------------------------------------------- stochastic: exact

def _one_child_tree(y):
    t = otree.verify_arrays(np.array([0, y], np.int32), np.array([-1, 0], np.int32),
                            np.array([0, 1], np.int32), np.ones(2, np.float32),
                            np.array([0, -1], np.int32), 0, 0)
    return {k: v[None] for k, v in t.items()}


def _first_token(p, q, y, ka, kd):
    V = len(p)
    t = _one_child_tree(y)
    prow = np.stack([np.asarray(p, np.float32), np.full(V, 1.0 / V, np.float32)])[None]
    u_acc = np.array([[0.0, ka * 2.0 ** -24]], np.float32)
    u_draw = np.array([[kd * 2.0 ** -24, 0.0]], np.float32)
    r = oacc.verify_stochastic(t, prow, np.asarray(q, np.float32)[None, None], u_acc, u_draw, S=1)
    return int(r["commit_tokens"][0, 0]), int(r["accept_len"][0])


def _first_monotone_change(f, lo, hi):
    """Least x in (lo, hi] with f(x) != f(lo) for a monotone step function f
    (once it leaves f(lo) it never returns); hi + 1 if none."""
    base = f(lo)
    if f(hi) == base:
        return hi + 1
    a, b = lo, hi
    while b - a > 1:
        m = (a + b) // 2
        if f(m) == base:
            a = m
        else:
            b = m
    return b


def enumerate_first_token(p, q_exact, y_support):
    """Exact P(first committed token = v), y ~ q (rational), all 2**24 x 2**24
    uniform pairs, using that acceptance is monotone in u_accept and the draw
    is monotone in u_draw (both follow from the sampling contract)."""
    V = len(p)
    q32 = np.array([float(x) for x in q_exact], np.float32)
    tot = {v: Fraction(0) for v in range(V)}
    n = 1 << 24
    for y in y_support:
        n_acc = _first_monotone_change(lambda ka: _first_token(p, q32, y, ka, 0)[1], 0, n - 1)
        if _first_token(p, q32, y, 0, 0)[1] == 0:
            n_acc = 0
        # the draw after a rejection: boundaries of the non-decreasing token map
        counts = {}
        if n_acc < n:
            ka = n_acc
            lo = 0
            while lo < n:
                v = _first_token(p, q32, y, ka, lo)[0]
                nxt = _first_monotone_change(lambda kd: _first_token(p, q32, y, ka, kd)[0], lo, n - 1)
                counts[v] = counts.get(v, 0) + (nxt - lo)
                lo = nxt
        w = Fraction(q_exact[y])
        tot[y] += w * Fraction(n_acc, n)
        for v, c in counts.items():
            tot[v] += w * Fraction(n - n_acc, n) * Fraction(c, n)
    return tot


def test_page_two_token_example_exact(golden_dir):
    g = _golden(golden_dir, "stochastic_two_token.json")
    q = [Fraction(4, 5), Fraction(1, 5)]
    tot = enumerate_first_token(g["p"], q, [0, 1])
    assert tot[0] == Fraction(*g["expected"]["0"])
    assert tot[1] == Fraction(*g["expected"]["1"])


def test_planted_resample_from_p_is_caught(golden_dir, monkeypatch):
    """Planting the page's wrong variant (redraw from p after a rejection) in
    the oracle moves the output distribution to 14/25, 11/25."""
    g = _golden(golden_dir, "stochastic_two_token.json")
    monkeypatch.setattr(oacc, "_rejection_draw_masses", lambda p_u, t, last: oacc.masses(p_u))
    tot = enumerate_first_token(g["p"], [Fraction(4, 5), Fraction(1, 5)], [0, 1])
    assert tot[0] != Fraction(*g["expected"]["0"])
    assert abs(float(tot[0]) - 14 / 25) < 1e-6
    assert abs(float(tot[1]) - 11 / 25) < 1e-6


@pytest.mark.parametrize("p,q", [
    ([Fraction(1, 4), Fraction(1, 2), Fraction(1, 4)], [Fraction(1, 2), Fraction(1, 4), Fraction(1, 4)]),
    ([Fraction(3, 8), Fraction(5, 8)], [Fraction(1, 2), Fraction(1, 2)]),
    ([Fraction(1, 16), Fraction(7, 16), Fraction(5, 16), Fraction(3, 16)],
     [Fraction(1, 4), Fraction(1, 4), Fraction(1, 4), Fraction(1, 4)]),
    ([Fraction(0), Fraction(1, 2), Fraction(1, 2)], [Fraction(1, 2), Fraction(0), Fraction(1, 2)]),
    ([Fraction(1, 2), Fraction(1, 2), Fraction(0)], [Fraction(1, 4), Fraction(1, 4), Fraction(1, 2)]),
])
def test_rejection_sampling_preserves_p_dyadic(p, q):
    """Dyadic p, power-of-two q: the sampled first token is distributed exactly as p."""
    support = [y for y in range(len(q)) if q[y] > 0]
    tot = enumerate_first_token([float(x) for x in p], q, support)
    assert [tot[v] for v in range(len(p))] == list(p)


def test_rejection_sampling_preserves_p_random_within_quantisation():
    rng = np.random.default_rng(11)
    for _ in range(3):
        V = 4
        p = workloads.softmax_rows(rng.standard_normal((1, V)).astype(np.float32) * 2)[0]
        q = workloads.softmax_rows(rng.standard_normal((1, V)).astype(np.float32) * 2)[0]
        qf = [Fraction(float(x)) for x in q]
        s = sum(qf)
        qf = [x / s for x in qf]
        tot = enumerate_first_token(p, qf, list(range(V)))
        for v in range(V):
            assert abs(float(tot[v]) - float(p[v])) < 1e-6


def test_sampling_primitives():
    # masses are exact fixed point; S sums in any order
    r = np.array([0.5, 2.0 ** -30, 0.25, 0.0], np.float32)
    R = oacc.masses(r)
    assert R.tolist() == [1 << 39, 1 << 10, 1 << 38, 0]
    # draw: T = floor(kk * S / 2**24); least i whose running mass exceeds T
    R = np.array([3, 0, 5], np.uint64)
    assert oacc.inverse_cdf(R, 0.0) == 0
    kk = (3 << 24) // 8                       # T = floor(kk * 8 / 2**24) = 3 -> index 2
    assert oacc.inverse_cdf(R, np.float32(kk * 2.0 ** -24)) == 2
    assert oacc.inverse_cdf(R, np.float32(((1 << 24) - 1) * 2.0 ** -24)) == 2
    # accept test is strict: u * q == t rejects
    assert not oacc.accept_test(np.float32(0.5), np.float32(0.8), np.float32(0.4))
    assert oacc.accept_test(np.float32(0.5 - 2 ** -24), np.float32(0.8), np.float32(0.4))


# ------------------------------------- stochastic: siblings (tree, k = 2)
#
# The walk's treatment of several children -- try them in sibling order, each
# rejection replacing t by the normalised residual (t - q)+ with q fixed, the
# correction drawn from the last residual -- is the multi-candidate
# ("multi-step") speculative sampling of SpecInfer (Miao et al., 2023).  Its
# theorem: when the candidates are drawn i.i.d. from q the committed token is
# distributed exactly as p.  The exact enumeration below feeds the oracle every
# pair (y1, y2) of i.i.d. draws as a two-child tree and every uniform.

def _two_child_tree(y1, y2):
    t = otree.verify_arrays(np.array([0, y1, y2], np.int32), np.array([-1, 0, 0], np.int32),
                            np.array([0, 1, 1], np.int32), np.ones(3, np.float32),
                            np.array([0, -1, -1], np.int32), 0, 0)
    return {k: v[None] for k, v in t.items()}


def _first_token_two(p, q32, y1, y2, ka1, ka2, kd):
    V = len(p)
    t = _two_child_tree(y1, y2)
    flat = np.full(V, 1.0 / V, np.float32)
    prow = np.stack([np.asarray(p, np.float32), flat, flat])[None]
    u_acc = np.array([[0.0, ka1 * 2.0 ** -24, ka2 * 2.0 ** -24]], np.float32)
    u_draw = np.array([[kd * 2.0 ** -24, 0.0, 0.0]], np.float32)
    r = oacc.verify_stochastic(t, prow, q32[None, None], u_acc, u_draw, S=1)
    return int(r["commit_tokens"][0, 0]), int(r["accept_path"][0, 1])


def enumerate_first_token_two(p, q_exact):
    """Exact P(first committed token = v) with y1, y2 ~ q i.i.d. and all
    uniforms; acceptance of each child is monotone in its own uniform and the
    draw is monotone in u_draw (sampling contract)."""
    V = len(p)
    q32 = np.array([float(x) for x in q_exact], np.float32)
    n = 1 << 24
    tot = {v: Fraction(0) for v in range(V)}
    support = [y for y in range(V) if q_exact[y] > 0]
    for y1 in support:
        for y2 in support:
            w = Fraction(q_exact[y1]) * Fraction(q_exact[y2])
            f1 = lambda ka: _first_token_two(p, q32, y1, y2, ka, n - 1, 0)[1] == 1   # noqa: E731
            n1 = 0 if not f1(0) else _first_monotone_change(f1, 0, n - 1)
            tot[y1] += w * Fraction(n1, n)
            if n1 == n:
                continue
            w1 = w * Fraction(n - n1, n)
            f2 = lambda ka: _first_token_two(p, q32, y1, y2, n1, ka, 0)[1] == 2     # noqa: E731
            n2 = 0 if not f2(0) else _first_monotone_change(f2, 0, n - 1)
            tot[y2] += w1 * Fraction(n2, n)
            if n2 == n:
                continue
            w2 = w1 * Fraction(n - n2, n)
            lo = 0
            while lo < n:
                v = _first_token_two(p, q32, y1, y2, n1, n2, lo)[0]
                nxt = _first_monotone_change(lambda kd: _first_token_two(p, q32, y1, y2, n1, n2, kd)[0], lo, n - 1)
                tot[v] += w2 * Fraction(nxt - lo, n)
                lo = nxt
    return tot


_SIBLING_CASES = [
    ([Fraction(1, 4), Fraction(1, 2), Fraction(1, 4)], [Fraction(1, 2), Fraction(1, 4), Fraction(1, 4)]),
    ([Fraction(1, 16), Fraction(7, 16), Fraction(5, 16), Fraction(3, 16)],
     [Fraction(1, 4), Fraction(1, 4), Fraction(1, 4), Fraction(1, 4)]),
    ([Fraction(2, 5), Fraction(3, 5)], [Fraction(4, 5), Fraction(1, 5)]),
    # residual above q on two tokens: skipping the normalisation would matter here
    ([Fraction(5, 8), Fraction(3, 8), Fraction(0), Fraction(0)],
     [Fraction(1, 8), Fraction(1, 8), Fraction(1, 4), Fraction(1, 2)]),
]


@pytest.mark.parametrize("p,q", _SIBLING_CASES)
def test_two_siblings_iid_from_q_preserve_p(p, q):
    """Within the contract's 2**-24 / 2**-40 quantisation (normalised residuals
    are rounded to fp32), the committed token of the two-sibling walk is p."""
    tot = enumerate_first_token_two([float(x) for x in p], q)
    assert sum(tot.values()) == 1
    for v in range(len(p)):
        assert abs(float(tot[v]) - float(p[v])) < 1e-6


def test_two_siblings_unnormalised_residual_is_caught(monkeypatch):
    """Planting a mistake in the oracle -- the next sibling tested against the
    raw residual instead of the normalised one -- moves the distribution."""
    p, q = _SIBLING_CASES[3]
    monkeypatch.setattr(oacc, "normalise", lambda r, S: np.asarray(r, np.float32))
    tot = enumerate_first_token_two([float(x) for x in p], q)
    assert max(abs(float(tot[v]) - float(p[v])) for v in range(len(p))) > 1e-3


# --------------------------------------------------- stochastic invariants

def test_stochastic_invariants_on_configs():
    for name in ("c2", "c4"):
        cfg = workloads.get_config(name, V=300, B=6)
        inp = workloads.generate(cfg, with_attention=False)
        # plant agreement so that walks go deep: p rows = q rows of the parent
        tp, ti = otopk.draft_topk(inp["draft_probs"], cfg.k)
        t = otree.build_tree(tp, ti, inp["root_token"], inp["prefix_len"], cfg.k, cfg.S, cfg.N)
        for planted in (False, True):
            p = inp["target"].copy()
            if planted:
                for b in range(cfg.B):
                    for u in range(cfg.N):
                        if t["q_row"][b, u] >= 0:
                            p[b, u] = inp["draft_probs"][b, t["q_row"][b, u]]
            r = oacc.verify_stochastic(t, p, inp["draft_probs"], inp["u_accept"], inp["u_draw"], S=cfg.S)
            for b in range(cfg.B):
                a = r["accept_len"][b]
                path = r["accept_path"][b, :a + 1]
                assert r["commit_len"][b] == a + 1
                assert path[0] == 0
                for d in range(1, a + 1):
                    assert t["parent"][b, path[d]] == path[d - 1]
                    assert r["commit_tokens"][b, d - 1] == t["tokens"][b, path[d]]
                assert r["next_root"][b] == r["commit_tokens"][b, a]
            if planted:
                assert r["accept_len"].mean() > 1


# ------------------------------- stochastic: the bonus after full acceptance
#
# A one-child chain root -> y, where y is a leaf.  If y is accepted, the walk
# draws the bonus at y from the target row there, p_leaf (zero-to-sglang ch.10
# section 5.1: after every draft token is accepted, one more token is sampled
# from the target distribution).  The enumeration covers every y ~ q, every
# u_accept, the correction draw at the root and the bonus draw at the leaf, and
# gives the exact law of the whole committed sequence.

def _walk_chain(p_root, p_leaf, q32, y, ka, kd_root, kd_leaf):
    V = len(p_root)
    t = _one_child_tree(y)
    prow = np.stack([np.asarray(p_root, np.float32), np.asarray(p_leaf, np.float32)])[None]
    u_acc = np.array([[0.0, ka * 2.0 ** -24]], np.float32)
    u_draw = np.array([[kd_root * 2.0 ** -24, kd_leaf * 2.0 ** -24]], np.float32)
    r = oacc.verify_stochastic(t, prow, q32[None, None], u_acc, u_draw, S=1)
    return tuple(int(x) for x in r["commit_tokens"][0, :r["commit_len"][0]])


def _draw_counts(f, n):
    """Counts of each value of a non-decreasing step function f over [0, n)."""
    counts, lo = {}, 0
    while lo < n:
        v = f(lo)
        nxt = _first_monotone_change(f, lo, n - 1)
        counts[v] = counts.get(v, 0) + (nxt - lo)
        lo = nxt
    return counts


def enumerate_chain_sequences(p_root, p_leaf, q_exact):
    """Exact law of the committed sequence of the one-child chain, y ~ q."""
    q32 = np.array([float(x) for x in q_exact], np.float32)
    n = 1 << 24
    law = {}
    for y in range(len(q_exact)):
        if q_exact[y] == 0:
            continue
        acc = lambda ka: len(_walk_chain(p_root, p_leaf, q32, y, ka, 0, 0)) == 2      # noqa: E731
        n_acc = 0 if not acc(0) else _first_monotone_change(acc, 0, n - 1)
        w = Fraction(q_exact[y])
        if n_acc > 0:
            bonus = _draw_counts(lambda kd: _walk_chain(p_root, p_leaf, q32, y, 0, 0, kd)[1], n)
            for v, c in bonus.items():
                law[(y, v)] = law.get((y, v), 0) + w * Fraction(n_acc, n) * Fraction(c, n)
        if n_acc < n:
            corr = _draw_counts(lambda kd: _walk_chain(p_root, p_leaf, q32, y, n_acc, kd, 0)[0], n)
            for v, c in corr.items():
                law[(v,)] = law.get((v,), 0) + w * Fraction(n - n_acc, n) * Fraction(c, n)
    return law


_BONUS_CASE = dict(
    p_root=[Fraction(1, 4), Fraction(1, 2), Fraction(1, 8), Fraction(1, 8)],
    # residual (p_root - q)+ = [0, 1/8, 0, 1/8]: its normalisation is dyadic,
    # so the 2**-24 uniforms reproduce every probability exactly
    q=[Fraction(1, 2), Fraction(3, 8), Fraction(1, 8), Fraction(0)],
    # the leaf's own target row differs from both p_root and q
    p_leaf=[Fraction(1, 16), Fraction(1, 8), Fraction(5, 16), Fraction(1, 2)],
)


def _expected_chain_law(p_root, q, p_leaf):
    """Speculative sampling with one candidate: y is committed with probability
    min(p(y), q(y)) and is followed by a bonus ~ p_leaf; otherwise the single
    token v is committed with probability p(v) - min(p(v), q(v))."""
    law = {}
    for y in range(len(q)):
        for v in range(len(p_leaf)):
            if min(p_root[y], q[y]) * p_leaf[v] > 0:
                law[(y, v)] = min(p_root[y], q[y]) * p_leaf[v]
    for v in range(len(p_root)):
        if p_root[v] - min(p_root[v], q[v]) > 0:
            law[(v,)] = p_root[v] - min(p_root[v], q[v])
    return law


def test_bonus_after_full_acceptance_is_drawn_from_the_leaf_row():
    c = _BONUS_CASE
    law = enumerate_chain_sequences([float(x) for x in c["p_root"]], [float(x) for x in c["p_leaf"]], c["q"])
    assert law == _expected_chain_law(c["p_root"], c["q"], c["p_leaf"])
    # the marginal of the first token is p_root, and given acceptance of y the
    # second token is distributed as p_leaf
    first = {}
    for seq, w in law.items():
        first[seq[0]] = first.get(seq[0], 0) + w
    assert [first.get(v, 0) for v in range(4)] == c["p_root"]


@pytest.mark.parametrize("plant", ["from_q", "from_parent_p"])
def test_planted_bonus_source_is_caught(monkeypatch, plant):
    """Planting a wrong bonus source in the oracle -- the draft row that
    proposed the leaf, or the parent's target row -- changes the exact law."""
    c = _BONUS_CASE
    p_root32 = np.array([float(x) for x in c["p_root"]], np.float32)
    if plant == "from_q":
        monkeypatch.setattr(oacc, "_leaf_bonus_masses", lambda p_leaf, q_parent: oacc.masses(q_parent))
    else:
        monkeypatch.setattr(oacc, "_leaf_bonus_masses", lambda p_leaf, q_parent: oacc.masses(p_root32))
    law = enumerate_chain_sequences([float(x) for x in c["p_root"]], [float(x) for x in c["p_leaf"]], c["q"])
    assert law != _expected_chain_law(c["p_root"], c["q"], c["p_leaf"])


def test_bonus_at_a_childless_root_is_drawn_from_p():
    """A root with no children (N = 1) commits one token drawn from its p row;
    every u_draw value is enumerated."""
    p = [Fraction(3, 8), Fraction(1, 8), Fraction(1, 2)]
    tree = otree.verify_arrays(np.array([0], np.int32), np.array([-1], np.int32), np.array([0], np.int32),
                               np.ones(1, np.float32), np.array([-1], np.int32), 0, 0)
    tree = {k: v[None] for k, v in tree.items()}
    prow = np.array([[float(x) for x in p]], np.float32)[None]

    def tok(kd):
        r = oacc.verify_stochastic(tree, prow, np.full((1, 1, 3), 1 / 3, np.float32),
                                   np.zeros((1, 1), np.float32), np.array([[kd * 2.0 ** -24]], np.float32), S=0)
        assert r["accept_len"][0] == 0 and r["commit_len"][0] == 1
        return int(r["commit_tokens"][0, 0])

    counts = _draw_counts(tok, 1 << 24)
    assert [Fraction(counts.get(v, 0), 1 << 24) for v in range(3)] == p


# ------------------------------------- the sampling contract at its edges
#
# tests/_sampling_edges.py builds requests that sit on the edges of the
# fixed-point contract; each carries a fact derived with exact rational or
# integer arithmetic (not with the oracle).  The oracle's walk must agree with
# every fact; the GPU test feeds the same batch to the kernel.

def _edge_batch():
    import _sampling_edges as edges
    return edges, *edges.build()


def test_sampling_edge_facts_hold_in_exact_arithmetic():
    """The constructions are sharp: the midpoint cases' S are realised by the
    rows' masses, and the draw facts follow from T = floor(kk * S / 2^24)."""
    edges, inp, cases = _edge_batch()
    for b, c in enumerate(cases):
        p0 = inp["target"][b, 0].astype(np.float64)
        if "S" in c:
            q = inp["draft_probs"][b, 0]
            r = np.maximum(inp["target"][b, 0] - q, np.float32(0))
            S = int(np.floor(r.astype(np.float64) * 2.0 ** 40).astype(np.uint64).sum(dtype=np.uint64))
            assert S == c["S"], c["name"]
            lo, hi = c["neighbours"]
            assert c["t_prime"] in (lo, hi) and lo < edges.U_MAX * hi < hi
        if "token" in c and not c["name"].startswith("masses below"):
            kk = int(round(float(inp["u_draw"][b, 0]) * (1 << 24)))
            m = np.floor(p0 * 2.0 ** 40).astype(np.int64)        # q is 0 wherever p is not
            S = int(sum(int(x) for x in m))
            T = kk * S >> 24
            cum = np.cumsum(m.astype(object))
            assert int(np.argmax(cum > T)) == c["token"], c["name"]
            if c["name"].startswith("crossing"):
                assert cum[c["token"] - 1] == T           # the running mass meets T exactly


def test_oracle_walk_agrees_with_the_edge_facts():
    edges, inp, cases = _edge_batch()
    tree = {k: inp[k] for k in ("tokens", "next_token", "next_sibling", "q_row")}
    r = oacc.verify_stochastic(tree, inp["target"], inp["draft_probs"], inp["u_accept"], inp["u_draw"], S=1)
    for b, c in enumerate(cases):
        name = c["name"]
        if name == "u*q == t rejects":
            assert r["accept_path"][b, 1] == 2                    # y1 rejected, y2 accepted
            assert r["commit_tokens"][b, :2].tolist() == [12, inp["target"].shape[2] - 1]
        elif name == "largest u accepts t == q":
            assert r["accept_path"][b, :2].tolist() == [0, 1] and r["commit_tokens"][b, 1] == 5
        elif "S" in c:
            q = inp["draft_probs"][b, 0]
            rr = np.maximum(inp["target"][b, 0] - q, np.float32(0))
            y2 = int(inp["tokens"][b, 2])
            assert float(oacc.normalise(rr, c["S"])[y2]) == c["t_prime"], name
            assert (r["accept_len"][b] == 1) == c["second_accepted"], name
        else:
            assert r["accept_len"][b] == 0 and r["commit_len"][b] == 1, name
            assert r["commit_tokens"][b, 0] == c["token"], name
