"""A batch of stochastic-accept requests built to sit on the edges of the
sampling arithmetic the accept walk fixes (zero-to-sglang ch.10 section 5.1,
with the fixed-point contract that makes it exact):

* accept iff fl64(u) * fl64(q[y]) < fl64(t[y]) -- equality rejects, the
  largest uniform (2^24 - 1) * 2^-24 accepts t == q;
* residual masses floor(r * 2^40): entries below 2^-40 have none, a level
  whose mass is zero keeps t, a draw with zero mass takes the argmax;
* normalised residual t' = fl32(fl64(r) / (fl64(S) * 2^-40)): cases whose
  fp64 quotient is an fp32 rounding midpoint exactly, or one fp64 ulp to
  either side of one, and one where S (near 2^56) is not representable in
  fp64 and rounding S down instead of to nearest flips the outcome;
* the draw T = floor(kk * S / 2^24), token = least i with a running mass
  above T: crossings exactly at T, on a boundary of the vocabulary slices the
  kernel splits a row into, kk = 0 and kk = 2^24 - 1, S below 2^24 and S
  near 2^57.

Every request is a root with up to two children (N = 3, S = 1, one draft
row); ``build(V)`` returns the tree arrays, the rows and the uniforms, and a
list of cases with the facts that make each one sharp (checked on the CPU
with exact rational arithmetic).  This module holds inputs only: what the
walk then commits is the oracle's to say.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

U_MAX = ((1 << 24) - 1) * 2.0 ** -24


def f32(x) -> float:
    return float(np.float32(x))


def up32(x: float) -> float:
    return float(np.nextafter(np.float32(x), np.float32(np.inf)))


def exact_t_prime(r: float, S: int) -> float:
    """The contract's normalised residual by exact arithmetic: the fp64
    quotient correctly rounded (Fraction -> float), then fp32 RNE."""
    return f32(float(Fraction(r) * 2 ** 40 / Fraction(float(S))))


def _fill_masses(total: int):
    """fp32 values in [0, 1] whose masses floor(v * 2^40) sum to ``total``
    exactly: ones, then one value with bits 16..39 and one with bits 0..15."""
    n1, rem = divmod(total, 1 << 40)
    vals = [1.0] * n1
    hi, lo = rem >> 16 << 16, rem & 0xFFFF
    for m in (hi, lo):
        if m:
            v = m * 2.0 ** -40
            assert f32(v) == v and int(v * 2 ** 40) == m
            vals.append(v)
    return vals


def _midpoint_case(kind: str, r2: float = 0.75, offset=0):
    """An S for which the second sibling's test separates the two fp32
    neighbours of a midpoint.  kind: 'tie' (fp64 quotient == midpoint, the
    even neighbour differs from the exact quotient's side), 'above' / 'below'
    (one fp64 ulp off the midpoint, the even neighbour on the other side),
    'u64' (S not representable; rounding S down would flip the result)."""
    for j in range(offset, offset + 400):
        c = f32(r2 * 2.0 ** -16 * (1 + j * 7.3e-4))
        cu = up32(c)
        M = (Fraction(c) + Fraction(cu)) / 2
        even_is_c = (int(np.float32(c).view(np.uint32)) & 1) == 0
        S0 = int(Fraction(r2) * 2 ** 40 / M)
        for S in range(S0 - 600, S0 + 600):
            fs = float(S)
            X = Fraction(r2) * 2 ** 40 / Fraction(fs)
            x64 = float(X)
            d = (Fraction(x64) - M) / Fraction(float(np.spacing(x64)))
            tp = exact_t_prime(r2, S)
            if kind == "tie" and d == 0 and S == int(fs):
                # single rounding of the exact quotient would go to X's side
                single = c if X < M else cu
                if (c if even_is_c else cu) != single:
                    return dict(S=S, c=c, cu=cu, t=tp, note="fp64 quotient is the fp32 midpoint: ties to even")
            if kind == "above" and d == 1 and S == int(fs) and even_is_c:
                return dict(S=S, c=c, cu=cu, t=tp, note="one fp64 ulp above the midpoint: rounds up")
            if kind == "below" and d == -1 and S == int(fs) and not even_is_c:
                return dict(S=S, c=c, cu=cu, t=tp, note="one fp64 ulp below the midpoint: rounds down")
            if kind == "u64" and S != int(fs) and int(fs) > S:
                trunc = Fraction(r2) * 2 ** 40 / Fraction(float(S - (S % int(np.spacing(fs)))))
                if f32(float(trunc)) != tp and abs(d) <= 2:
                    return dict(S=S, c=c, cu=cu, t=tp, note="S rounds up to fp64; truncating it flips t'")
    raise RuntimeError("no %s case found" % kind)


def build(V: int = 128256):
    cases = []
    rows = []          # per request: (p rows [3, V], q row [V], tree dict, u_accept[3], u_draw[3])

    def new_rows():
        return np.zeros((3, V), np.float32), np.zeros(V, np.float32)

    def tree(kids):
        tok = [0, 0, 0]
        nxt, sib, qr = [-1, -1, -1], [-1, -1, -1], [-1, -1, -1]
        if kids:
            nxt[0], qr[0] = 1, 0
            tok[1] = kids[0]
            if len(kids) > 1:
                tok[2] = kids[1]
                sib[1] = 2
        return dict(tokens=tok, next_token=nxt, next_sibling=sib, q_row=qr)

    def add(name, p, q, kids, ua, ud, **facts):
        cases.append(dict(name=name, **facts))
        rows.append((p, q, tree(kids), [0.0] + list(ua) + [0.0] * (2 - len(ua)), list(ud)))

    # accept test equality rejects; the largest uniform accepts t == q; the
    # bonus at the leaf crosses at the row's last entry
    p, q = new_rows()
    y1, y2 = 11, 12
    p[0, : 1 << 17] = 2.0 ** -18
    p[0, y1], p[0, y2] = f32(0.4), f32(0.1)
    q[y1], q[y2] = f32(0.8), f32(0.05)
    p[2, 0], p[2, V - 1] = 0.5, 0.5
    assert float(np.float32(0.5)) * float(q[y1]) == float(p[0, y1])
    add("u*q == t rejects", p, q, [y1, y2], [0.5, U_MAX], [0.0, 0.0, U_MAX])

    p, q = new_rows()
    p[0, 77], q[77] = f32(0.3), f32(0.3)
    p[1, 5], p[1, 9] = 0.25, 0.75
    add("largest u accepts t == q", p, q, [77], [U_MAX], [0.0, 0.0, 0.0])

    # the second sibling's test against a near-midpoint normalised residual
    y1, y2 = 100000, 60001
    for kind, off in (("tie", 0), ("above", 0), ("below", 0), ("u64", 0)):
        mc = _midpoint_case(kind, offset=off)
        p, q = new_rows()
        q[y1] = 1.0                                # p[y1] = 0: y1 is always rejected
        Q2 = mc["cu"]
        P2 = f32(0.75 + Q2)
        assert f32(P2 - Q2) == 0.75
        q[y2], p[0, y2] = Q2, P2
        fill = _fill_masses(mc["S"] - int(0.75 * 2 ** 40))
        idx = [i for i in range(V) if i not in (y1, y2)][: len(fill)]
        p[0, idx] = np.asarray(fill, np.float32)
        p[2, 3] = 1.0
        accept = U_MAX * Q2 < mc["t"]
        add("t' " + kind, p, q, [y1, y2], [0.5, U_MAX], [0.3, 0.0, 0.0],
            S=mc["S"], t_prime=mc["t"], neighbours=(mc["c"], mc["cu"]), second_accepted=accept, why=mc["note"])

    # exact crossings of the draw: at a slice boundary (index 2^15) and inside
    for kk, want in ((1 << 23, 32768), ((1 << 23) + 3 * 256, 32771)):
        p, q = new_rows()
        q[100000] = 1.0
        p[0, : 1 << 16] = 2.0 ** -16               # masses 2^24, S = 2^40
        add("crossing T == running mass, kk=%d" % kk, p, q, [100000], [0.5], [kk * 2.0 ** -24, 0.0, 0.0],
            token=want)

    # masses below 2^-40: both levels have S = 0 (t kept), the draw has zero
    # mass and takes the argmax (lowest id among equals)
    p, q = new_rows()
    p[0, :] = 2.0 ** -41
    p[0, 7] = p[0, 9] = 3 * 2.0 ** -42
    q[5] = q[6] = 1.0
    add("masses below 2^-40", p, q, [5, 6], [0.25, 0.25], [0.7, 0.0, 0.0], token=7)

    # kk = 0 at a childless root: the first entry of positive mass
    p, q = new_rows()
    p[0, 1000] = 2.0 ** -41
    p[0, 50000] = 2.0 ** -40
    p[0, 50001] = 0.5
    add("kk = 0", p, q, [], [], [0.0, 0.0, 0.0], token=50000)

    # S below 2^24 with kk = 2^24 - 1
    p, q = new_rows()
    p[0, 3] = 5 * 2.0 ** -40
    p[0, 70000] = 2.0 ** -20
    add("S < 2^24, kk = 2^24 - 1", p, q, [], [], [U_MAX, 0.0, 0.0], token=70000)

    # S near 2^57 with low bits set, kk = 2^24 - 1: the last entry
    p, q = new_rows()
    p[0, :] = 1.0
    p[0, 0] = f32(1.0 - 2.0 ** -24)
    add("S near 2^57", p, q, [], [], [U_MAX, 0.0, 0.0], token=V - 1)

    B = len(rows)
    out = dict(
        target=np.stack([r[0] for r in rows]),
        draft_probs=np.stack([r[1] for r in rows])[:, None, :],
        u_accept=np.array([r[3] for r in rows], np.float32),
        u_draw=np.array([r[4] for r in rows], np.float32),
    )
    for key in ("tokens", "next_token", "next_sibling", "q_row"):
        out[key] = np.array([r[2][key] for r in rows], np.int32)
    assert out["target"].shape == (B, 3, V)
    return out, cases
