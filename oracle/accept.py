"""Oracle: the accept walk over a verified tree (greedy and rejection sampling).

Follows zero-to-sglang ch.10:
* section 3.3 -- the target row of a position verifies the token after it; the
  row after the last draft token picks the bonus token;
* section 4.1 -- ``greedy_commit``: take the target's choice per row, commit it,
  stop at the first mismatch, at EOS or when the output budget is used up;
  after a full match the last row adds a bonus token; budget 0 commits nothing;
* section 4.2 -- worked example: draft [1,1,1], target picks 1 then 2 ->
  [1, 2] is committed;
* section 5.1 -- rejection sampling: accept a candidate y with probability
  min(1, p[y]/q[y]); on rejection draw from the normalised positive residual
  (p - q)+; stop at the first rejection; after full acceptance draw the bonus
  from p; p and q are the processed distributions actually sampled from.
"EAGLE speculative decoding in four parts", "Drafting, verification and
slots": the verification kernels walk the tree to each request's longest
accepted path.  sglang PR #22883 ("Modifications"): the acceptance criterion
is unchanged under TLI.

Readings where the pages leave a step open:
* Target row u of request b is the target's distribution after tree node u
  (greedy: raw logits; stochastic: processed p).  The draft distribution that
  produced u's children is draft row q_row[u].
* Tree generalisation, greedy: sibling tokens are distinct, so at most one
  child of u carries the target's choice; the walk moves to it.
* Tree generalisation, stochastic: at node u, t := p_u; the children are tried
  in sibling order; a rejected child replaces t by the normalised residual
  (t - q_u)+ with q_u held fixed; the first accepted child is moved to; if all
  are rejected the correction is drawn from the last residual; at a leaf the
  bonus is drawn from p_u.  This is the multi-candidate speculative sampling
  of SpecInfer (Miao et al., 2023), which commits exactly p when the
  candidates are i.i.d. draws from q (pinned by exact enumeration); for the
  deterministic top-k children of a draft tree no output law is claimed.
* An EOS or budget stop on a token that matched a child counts that child as
  accepted, with no further token.
* Sampling arithmetic (makes the walk bit-exact across devices):
  - accept y iff fl64(u) * fl64(q[y]) < fl64(t[y])  (u has 24 bits: exact);
  - residual r_i = max(t_i - q_i, 0), one fp32 subtraction;
  - masses R_i = floor(r_i * 2**40) as unsigned 64-bit; S = sum R_i (exact);
  - normalised residual t'_i = fl32(fl64(r_i) / (fl64(S) * 2**-40));
  - draw with u = kk * 2**-24: T = floor(kk * S / 2**24), token = the least i
    with R_0 + .. + R_i > T;
  - if a residual has S = 0, t is kept; a draw whose masses sum to 0 takes the
    argmax of t (lowest id).
"""
from __future__ import annotations

import numpy as np

TWO40 = 2.0 ** 40


def children(next_token, next_sibling, u: int):
    """Children of node u in sibling order (ascending tree index)."""
    out = []
    c = int(next_token[u])
    while c >= 0:
        out.append(c)
        c = int(next_sibling[c])
    return out


def argmax_lowest(row) -> int:
    """Index of the largest value; the lowest index among equals."""
    return int(np.argmax(np.asarray(row)))


# ---------------------------------------------------------------- greedy

def _greedy_one(tokens, next_token, next_sibling, target_rows, eos_id, remaining):
    path, out = [0], []
    if remaining == 0:
        return path, out
    u = 0
    while True:
        t = argmax_lowest(target_rows[u])
        out.append(t)
        match = None
        for c in children(next_token, next_sibling, u):
            if int(tokens[c]) == t:
                match = c
                break
        if match is not None:
            path.append(match)
        if t == eos_id or (remaining is not None and len(out) == remaining) or match is None:
            return path, out
        u = match


# ------------------------------------------------------------ stochastic

def accept_test(u, q_y, t_y) -> bool:
    """Accept iff u * q[y] < t[y], evaluated in float64 (exact for 24-bit u)."""
    return float(np.float32(u)) * float(np.float32(q_y)) < float(np.float32(t_y))


def residual(t, q):
    """(t - q)+ as one fp32 subtraction per entry."""
    return np.maximum(np.asarray(t, np.float32) - np.asarray(q, np.float32), np.float32(0))


def masses(w):
    """Fixed-point masses floor(w * 2**40) of non-negative fp32 weights."""
    return np.floor(np.asarray(w, np.float32).astype(np.float64) * TWO40).astype(np.uint64)


def normalise(r, S: int):
    """fl32(fl64(r_i) / (fl64(S) * 2**-40))."""
    s = float(S) * 2.0 ** -40
    return (np.asarray(r, np.float32).astype(np.float64) / s).astype(np.float32)


def inverse_cdf(R, u) -> int:
    """Least i with R_0 + ... + R_i > floor(kk * S / 2**24), u = kk * 2**-24."""
    kk = int(round(float(np.float32(u)) * (1 << 24)))
    S = int(np.asarray(R, np.uint64).sum(dtype=np.uint64))
    assert 0 < S and 0 <= kk < (1 << 24)
    T = (kk * S) >> 24
    c = np.cumsum(np.asarray(R, np.uint64), dtype=np.uint64)
    return int(np.searchsorted(c, np.uint64(T), side="right"))


def _rejection_draw_masses(p_u, t, last):
    """Masses the correction is drawn from once every child is rejected."""
    return last


def _leaf_bonus_masses(p_leaf, q_parent):
    """Masses of the bonus drawn at a leaf: the target's own row at the leaf.

    q_parent (the draft row that proposed the leaf; None at a root without
    children) is not used: the bonus comes from p alone, not from q."""
    return masses(p_leaf)


def _draw(R, t, u) -> int:
    if int(np.asarray(R, np.uint64).sum(dtype=np.uint64)) == 0:
        return argmax_lowest(t)
    return inverse_cdf(R, u)


def _stochastic_one(b, tokens, next_token, next_sibling, q_row, p_rows, q_rows,
                    u_accept, u_draw, eos_id, remaining):
    path, out = [0], []
    if remaining == 0:
        return path, out
    u = 0
    q_parent = None
    while True:
        p_u = np.asarray(p_rows[u], np.float32)
        t = p_u
        kids = children(next_token, next_sibling, u)
        accepted, last = None, None
        if kids:
            q = np.asarray(q_rows[int(q_row[u])], np.float32)
            for c in kids:
                y = int(tokens[c])
                if accept_test(u_accept[c], q[y], t[y]):
                    accepted = c
                    break
                r = residual(t, q)
                R = masses(r)
                S = int(R.sum(dtype=np.uint64))
                if S > 0:
                    t = normalise(r, S)
                    last = R
                else:
                    last = masses(t)
        if accepted is not None:
            y = int(tokens[accepted])
            out.append(y)
            path.append(accepted)
            if y == eos_id or (remaining is not None and len(out) == remaining):
                return path, out
            u = accepted
            q_parent = q
            continue
        R = _rejection_draw_masses(p_u, t, last) if kids else _leaf_bonus_masses(p_u, q_parent)
        out.append(_draw(R, t, u_draw[u]))
        return path, out


# ------------------------------------------------------------------ batch

def _pack(results, B, S):
    accept_len = np.zeros(B, np.int32)
    accept_path = np.full((B, S + 1), -1, np.int32)
    commit_tokens = np.full((B, S + 1), -1, np.int32)
    commit_len = np.zeros(B, np.int32)
    next_root = np.full(B, -1, np.int32)
    for b, (path, out) in enumerate(results):
        accept_len[b] = len(path) - 1
        accept_path[b, :len(path)] = path
        commit_tokens[b, :len(out)] = out
        commit_len[b] = len(out)
        if out:
            next_root[b] = out[-1]
    return dict(accept_len=accept_len, accept_path=accept_path, commit_tokens=commit_tokens,
                commit_len=commit_len, next_root=next_root)


def verify_greedy(tree, target, S: int, eos_id: int = -1, remaining=None):
    """Greedy accept for a batch.

    tree: dict with tokens/next_token/next_sibling [B,N]; target [B,N,V] logits.
    remaining: None (unlimited) or [B] non-negative output budgets.
    Returns accept_len [B], accept_path [B,S+1] (root first, -1 pad),
    commit_tokens [B,S+1] (-1 pad), commit_len [B], next_root [B] (-1 if none).
    """
    B = tree["tokens"].shape[0]
    res = []
    for b in range(B):
        rem = None if remaining is None else int(remaining[b])
        res.append(_greedy_one(tree["tokens"][b], tree["next_token"][b], tree["next_sibling"][b],
                               target[b], eos_id, rem))
    return _pack(res, B, S)


def verify_stochastic(tree, p, draft_probs, u_accept, u_draw, S: int, eos_id: int = -1,
                      remaining=None):
    """Rejection-sampling accept for a batch.

    p [B,N,V] processed target rows; draft_probs [B,R,V] processed draft rows
    (row q_row[u] produced u's children); u_accept[b,c] decides child c,
    u_draw[b,u] is the one draw at node u.  Outputs as ``verify_greedy``.
    """
    B = tree["tokens"].shape[0]
    res = []
    for b in range(B):
        rem = None if remaining is None else int(remaining[b])
        res.append(_stochastic_one(b, tree["tokens"][b], tree["next_token"][b],
                                   tree["next_sibling"][b], tree["q_row"][b], p[b],
                                   draft_probs[b], u_accept[b], u_draw[b], eos_id, rem))
    return _pack(res, B, S)
