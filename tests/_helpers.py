"""Helpers shared by the GPU parity tests (host <-> device marshalling, the
test-only planting of accepted paths, and the tolerance check)."""
import numpy as np
import torch

from oracle import topk as otopk
from oracle import tree as otree


def dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def host(t):
    return t.detach().cpu().numpy()


def bf16_to_f64(t):
    """Device bf16 (or int16 bits) tensor -> float64 numpy."""
    if t.dtype != torch.bfloat16:
        t = t.view(torch.bfloat16)
    return t.float().cpu().numpy().astype(np.float64)


def oracle_tree(inp, cfg, draft_key="draft_probs"):
    tp, ti = otopk.draft_topk(inp[draft_key], cfg.k)
    return otree.build_tree(tp, ti, inp["root_token"], inp["prefix_len"], cfg.k, cfg.S, cfg.N)


def plant_greedy(target, tree, rng, S):
    """Make the target's argmax follow a random-length path of first children."""
    t = target.copy()
    B = t.shape[0]
    for b in range(B):
        a = int(rng.integers(0, S + 1))
        u = 0
        for _ in range(a):
            c = int(tree["next_token"][b, u])
            if c < 0:
                break
            t[b, u, tree["tokens"][b, c]] = t[b, u].max() + 1.0
            u = c
    return t


def plant_stochastic(p, draft, tree, rng, S):
    """Set the target row of the nodes on a random-length path to the draft row
    that produced their children, so those children are accepted for u < 1."""
    t = p.copy()
    B = t.shape[0]
    for b in range(B):
        a = int(rng.integers(0, S + 1))
        u = 0
        for _ in range(a):
            c = int(tree["next_token"][b, u])
            if c < 0 or tree["q_row"][b, u] < 0:
                break
            t[b, u] = draft[b, tree["q_row"][b, u]]
            u = c
    return t


def assert_attention_close(got, ref, max_abs=2e-2, rel=1e-2):
    """max |got - ref| <= max_abs and ||got - ref||_2 <= rel * ||ref||_2."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert np.isfinite(got).all()
    err = np.abs(got - ref)
    assert err.max() <= max_abs, "max abs error %g" % err.max()
    nrm = np.linalg.norm(ref)
    assert np.linalg.norm(got - ref) <= rel * nrm, "relative error %g" % (np.linalg.norm(got - ref) / nrm)
