"""Pins of the oracle's attention, compaction and TLI stages."""
import numpy as np
import pytest
import torch

from oracle import attention as oatt
from oracle import compact as ocmp
from oracle import tli as otli
from oracle import topk as otopk
from oracle import tree as otree
from oracle import accept as oacc
import workloads


def _bf(x):
    return workloads.to_bf16_bits(np.asarray(x, np.float32))


def _random_tree(rng, k, S, N, V=64):
    R = 1 + (S - 1) * k
    probs = workloads.softmax_rows(rng.standard_normal((1, R, V)).astype(np.float32) * 2)
    tp, ti = otopk.draft_topk(probs, k)
    return otree.build_tree(tp, ti, np.array([1]), np.array([0]), k, S, N)


def _layout(rng, logical_len, page):
    """Scatter logical positions of one request into a shuffled paged pool."""
    n_pages = -(-logical_len // page)
    total = n_pages + 3
    phys = rng.permutation(total)[:n_pages].astype(np.int32)
    return phys, total


def _pooled(rng, K_log, V_log, page):
    """Pool holding one request's logical K/V [T, Hkv, D] under a random page chain."""
    T = K_log.shape[0]
    phys, total = _layout(rng, T, page)
    kp = _bf(rng.standard_normal((total * page,) + K_log.shape[1:]))   # garbage elsewhere
    vp = _bf(rng.standard_normal((total * page,) + K_log.shape[1:]))
    for pos in range(T):
        s = phys[pos // page] * page + pos % page
        kp[s] = K_log[pos]
        vp[s] = V_log[pos]
    return kp, vp, phys[None]


@pytest.mark.parametrize("k,S,N,L,Hq,Hkv,D,page", [(2, 3, 6, 40, 4, 4, 64, 1), (4, 3, 12, 33, 8, 2, 32, 16),
                                                   (1, 4, 5, 17, 4, 1, 16, 4), (3, 3, 10, 0, 2, 2, 16, 1)])
def test_attention_equals_library_sdpa_on_each_path(k, S, N, L, Hq, Hkv, D, page):
    """Every node's output is ordinary attention over prefix + its root path
    (torch's scaled_dot_product_attention in float64)."""
    rng = np.random.default_rng(N * 7 + L)
    t = _random_tree(rng, k, S, N)
    K_log = _bf(rng.standard_normal((L + N, Hkv, D)))
    V_log = _bf(rng.standard_normal((L + N, Hkv, D)))
    q = _bf(rng.standard_normal((1, N, Hq, D)))
    kp, vp, table = _pooled(rng, K_log, V_log, page)
    out, lse = oatt.tree_verify_attention(q, kp, vp, table, np.array([L]), t["mask"], page=page)
    Kf = torch.from_numpy(workloads.bf16_bits_to_f32(K_log).astype(np.float64))
    Vf = torch.from_numpy(workloads.bf16_bits_to_f32(V_log).astype(np.float64))
    Qf = torch.from_numpy(workloads.bf16_bits_to_f32(q).astype(np.float64))
    G = Hq // Hkv
    for i in range(N):
        anc, j = [], i
        while j >= 0:
            anc.append(j)
            j = int(t["parent"][0, j])
        keys = list(range(L)) + [L + a for a in sorted(anc)]
        for h in range(Hq):
            kk = Kf[keys, h // G][None, None]
            vv = Vf[keys, h // G][None, None]
            ref = torch.nn.functional.scaled_dot_product_attention(Qf[0, i, h][None, None, None], kk, vv)
            assert np.allclose(out[0, i, h], ref[0, 0, 0].numpy(), rtol=1e-12, atol=1e-12)
            s = (kk[0, 0] @ Qf[0, i, h]) / np.sqrt(D)
            assert np.isclose(lse[0, i, h], torch.logsumexp(s, 0).item(), rtol=1e-12)


def test_attention_root_only_is_decode_attention():
    rng = np.random.default_rng(5)
    L, Hq, Hkv, D = 50, 4, 2, 32
    K_log = _bf(rng.standard_normal((L + 1, Hkv, D)))
    V_log = _bf(rng.standard_normal((L + 1, Hkv, D)))
    q = _bf(rng.standard_normal((1, 1, Hq, D)))
    kp, vp, table = _pooled(rng, K_log, V_log, 1)
    out, _ = oatt.tree_verify_attention(q, kp, vp, table, np.array([L]), np.ones((1, 1, 1), np.uint8))
    Kf = workloads.bf16_bits_to_f32(K_log).astype(np.float64)
    Vf = workloads.bf16_bits_to_f32(V_log).astype(np.float64)
    Qf = workloads.bf16_bits_to_f32(q).astype(np.float64)
    for h in range(Hq):
        kk = torch.from_numpy(Kf[:, h // 2])[None, None]
        vv = torch.from_numpy(Vf[:, h // 2])[None, None]
        ref = torch.nn.functional.scaled_dot_product_attention(torch.from_numpy(Qf[0, 0, h])[None, None, None], kk, vv)
        assert np.allclose(out[0, 0, h], ref[0, 0, 0].numpy(), atol=1e-12)


def test_attention_chain_is_causal_attention():
    """topk=1 chain: the tree mask is the causal mask over the appended tokens."""
    rng = np.random.default_rng(6)
    L, N, H, D = 20, 5, 2, 16
    t = _random_tree(rng, 1, N - 1, N)
    K_log = _bf(rng.standard_normal((L + N, H, D)))
    V_log = _bf(rng.standard_normal((L + N, H, D)))
    q = _bf(rng.standard_normal((1, N, H, D)))
    kp, vp, table = _pooled(rng, K_log, V_log, 1)
    out, _ = oatt.tree_verify_attention(q, kp, vp, table, np.array([L]), t["mask"])
    Kf = torch.from_numpy(workloads.bf16_bits_to_f32(K_log).astype(np.float64)).permute(1, 0, 2)
    Vf = torch.from_numpy(workloads.bf16_bits_to_f32(V_log).astype(np.float64)).permute(1, 0, 2)
    Qf = torch.from_numpy(workloads.bf16_bits_to_f32(q[0]).astype(np.float64)).permute(1, 0, 2)
    causal = torch.ones(N, L + N, dtype=torch.bool).tril(diagonal=L)
    ref = torch.nn.functional.scaled_dot_product_attention(Qf[None], Kf[None], Vf[None], attn_mask=causal)
    assert np.allclose(out[0], ref[0].permute(1, 0, 2).numpy(), atol=1e-12)


# ------------------------------------------------------------- compaction

def _compaction_case(rng, page, B=5, N=12, layers=2, Hkv=2, D=8):
    L = rng.integers(0, 40, size=B).astype(np.int32)
    need = (L + N + page - 1) // page
    total = int(need.sum()) + 4
    perm = rng.permutation(total).astype(np.int32)
    table = np.full((B, int(need.max()) + 1), -1, np.int32)
    off = 0
    for b in range(B):
        table[b, :need[b]] = perm[off:off + need[b]]
        off += need[b]
    kps = [rng.integers(0, 65535, size=(total * page, Hkv, D)).astype(np.uint16) for _ in range(layers)]
    vps = [rng.integers(0, 65535, size=(total * page, Hkv, D)).astype(np.uint16) for _ in range(layers)]
    S = 4
    acc_len = np.zeros(B, np.int32)
    acc_path = np.full((B, S + 1), -1, np.int32)
    for b in range(B):
        a = int(rng.integers(0, S + 1))
        path = [0] + sorted(rng.choice(np.arange(1, N), size=a, replace=False).tolist())
        acc_len[b] = a
        acc_path[b, :a + 1] = path
    return L, table, kps, vps, acc_len, acc_path, N


def test_compaction_page1_is_slot_remap():
    rng = np.random.default_rng(21)
    L, table, kps, vps, a, path, N = _compaction_case(rng, 1)
    t2, kp2, vp2, new_len, freed = ocmp.compact_kv(table, kps, vps, L, a, path, N, 1)
    freed_all = []
    for b in range(len(L)):
        tree_slots = table[b, L[b]:L[b] + N].tolist()
        kept = [table[b, L[b] + p] for p in path[b, :a[b] + 1]]
        assert t2[b, L[b]:L[b] + a[b] + 1].tolist() == kept
        assert (t2[b, L[b] + a[b] + 1:L[b] + N] == -1).all()
        assert np.array_equal(t2[b, :L[b]], table[b, :L[b]])          # prefix untouched
        assert new_len[b] == L[b] + a[b] + 1
        mine = [s for j, s in enumerate(tree_slots) if j not in set(path[b, :a[b] + 1].tolist())]
        assert set(mine) | set(kept) == set(tree_slots) and not set(mine) & set(kept)
        freed_all += mine
    assert freed.tolist() == freed_all
    for x, y in zip(kps + vps, kp2 + vp2):
        assert np.array_equal(x, y)                                      # no bytes move


@pytest.mark.parametrize("page", [4, 16])
def test_compaction_paged_moves_accepted_kv(page):
    rng = np.random.default_rng(22 + page)
    L, table, kps, vps, a, path, N = _compaction_case(rng, page)
    t2, kp2, vp2, new_len, freed = ocmp.compact_kv(table, kps, vps, L, a, path, N, page)

    def slot(b, pos):
        return table[b, pos // page] * page + pos % page

    exp_freed = []
    for b in range(len(L)):
        for d in range(a[b] + 1):
            for old, new in zip(kps + vps, kp2 + vp2):
                assert np.array_equal(new[slot(b, L[b] + d)], old[slot(b, L[b] + path[b, d])])
        for pos in range(L[b]):
            for old, new in zip(kps + vps, kp2 + vp2):
                assert np.array_equal(new[slot(b, pos)], old[slot(b, pos)])
        nl = L[b] + a[b] + 1
        assert new_len[b] == nl
        keep_pages = -(-nl // page)
        used_pages = (L[b] + N - 1) // page + 1
        assert np.array_equal(t2[b, :keep_pages], table[b, :keep_pages])
        assert (t2[b, keep_pages:used_pages] == -1).all()
        exp_freed += table[b, keep_pages:used_pages].tolist()
    assert freed.tolist() == exp_freed


def test_compaction_overlapping_moves():
    """path [0, 2, 3]: the copy into position 2 must read the old node 3 and
    the copy into position 1 the old node 2 (no read-after-write mix-up)."""
    page = 4
    L = np.array([2], np.int32)
    table = np.array([[0, 1, 2, 3]], np.int32)
    kp = [np.arange(16 * 1 * 1, dtype=np.uint16).reshape(16, 1, 1)]
    vp = [kp[0] + 100]
    t2, kp2, vp2, new_len, freed = ocmp.compact_kv(table, kp, vp, L, np.array([2]),
                                                  np.array([[0, 2, 3, -1]]), 7, page)
    assert kp2[0][2:5, 0, 0].tolist() == [2, 4, 5]
    assert vp2[0][2:5, 0, 0].tolist() == [102, 104, 105]
    assert new_len.tolist() == [5] and freed.tolist() == [2]


# ------------------------------------------------------------------- TLI

def _tli_case(rng, Vd=300, Vt=250, K=120):
    inter = np.sort(rng.choice(Vd, size=K, replace=False)).astype(np.int32)
    tgt = rng.choice(Vt, size=K, replace=False).astype(np.int32)
    outside = np.setdiff1d(np.arange(Vd), inter)
    return inter, tgt, int(outside[0])


def test_tli_maps_are_inverse_on_the_intersection():
    rng = np.random.default_rng(31)
    inter, tgt, fb = _tli_case(rng)
    d2t, t2d = otli.build_maps(inter, tgt, 300, 250, fb)
    assert np.array_equal(otli.map_ids(t2d, otli.map_ids(d2t, inter)), inter)
    assert np.array_equal(otli.map_ids(d2t, otli.map_ids(t2d, tgt)), tgt)
    outside_t = np.setdiff1d(np.arange(250), tgt)
    assert (otli.map_ids(t2d, outside_t) == fb).all()
    assert (otli.map_ids(d2t, np.setdiff1d(np.arange(300), inter)) == -1).all()
    assert otli.map_ids(d2t, np.array([300, -1, inter[0]])).tolist() == [-1, -1, tgt[0]]


def test_tli_pruned_head_equals_full_head_columns():
    rng = np.random.default_rng(32)
    inter, _, _ = _tli_case(rng)
    H = 48
    hidden = _bf(rng.standard_normal((7, H)))
    W_full = _bf(rng.standard_normal((300, H)) * 0.02)
    full = workloads.bf16_bits_to_f32(hidden).astype(np.float64) @ \
        workloads.bf16_bits_to_f32(W_full).astype(np.float64).T
    pruned = otli.lm_head(hidden, W_full[inter])
    assert np.allclose(pruned, full[:, inter], rtol=1e-13, atol=1e-15)


def test_tli_constrained_softmax_has_no_mass_outside():
    rng = np.random.default_rng(33)
    inter, _, _ = _tli_case(rng)
    pruned = rng.standard_normal((3, len(inter))).astype(np.float32)
    full = otli.constrain_logits(pruned, inter, 300)
    p = torch.softmax(torch.from_numpy(full.astype(np.float64)), dim=1).numpy()
    outside = np.setdiff1d(np.arange(300), inter)
    assert (p[:, outside] == 0).all()
    assert np.allclose(p[:, inter], torch.softmax(torch.from_numpy(pruned.astype(np.float64)), 1).numpy())


def test_tli_identity_vocab_reduces_to_plain_verify():
    """V_draft = V_target = K with the identity pairing: the scattered draft
    rows are the draft rows and the verify is the ordinary one."""
    cfg = workloads.get_config("c2", V=200, B=4)
    inp = workloads.generate(cfg, with_attention=False)
    ident = np.arange(cfg.V, dtype=np.int32)
    q2 = otli.q_scatter(inp["draft_probs"].reshape(-1, cfg.V), ident, cfg.V).reshape(inp["draft_probs"].shape)
    assert np.array_equal(q2, inp["draft_probs"])
    d2t, t2d = otli.build_maps(ident, ident, cfg.V, cfg.V, 0)
    assert np.array_equal(d2t, ident) and np.array_equal(t2d, ident)
    tp, ti = otopk.draft_topk(q2, 1)
    t = otree.build_tree(tp, ti, inp["root_token"], inp["prefix_len"], 1, cfg.S, cfg.N)
    r1 = oacc.verify_stochastic(t, inp["target"], q2, inp["u_accept"], inp["u_draw"], S=cfg.S)
    tp0, ti0 = otopk.draft_topk(inp["draft_probs"], 1)
    t0 = otree.build_tree(tp0, ti0, inp["root_token"], inp["prefix_len"], 1, cfg.S, cfg.N)
    r0 = oacc.verify_stochastic(t0, inp["target"], inp["draft_probs"], inp["u_accept"], inp["u_draw"], S=cfg.S)
    for key in r0:
        assert np.array_equal(r0[key], r1[key])


def test_tli_small_pairing_golden(golden_dir):
    import json
    import os
    with open(os.path.join(golden_dir, "tli_small_pairing.json")) as f:
        g = json.load(f)
    d2t, t2d = otli.build_maps(g["inter_ids"], g["tgt_ids"], g["V_draft"], g["V_target"], g["fallback"])
    assert d2t.tolist() == g["expected_d2t"]
    assert t2d.tolist() == g["expected_t2d"]
    q = otli.q_scatter(np.array([g["q_pruned"]], np.float32), g["tgt_ids"], g["V_target"])
    assert q[0].tolist() == g["expected_q_target"]


def _q_target_semantics_hold(q_target, q_dense, d2t, t2d):
    """Target id t carries the draft probability of its draft counterpart
    t2d[t] when that is an intersection token (d2t[t2d[t]] == t), else 0."""
    Vt = q_target.shape[1]
    for t in range(Vt):
        d = int(t2d[t])
        want = q_dense[:, d] if 0 <= d < len(d2t) and d2t[d] == t else np.zeros(q_dense.shape[0], np.float32)
        if not np.array_equal(q_target[:, t], want):
            return False
    return True


def _q_scatter_case():
    rng = np.random.default_rng(34)
    Vd, Vt, K = 300, 250, 120
    inter, tgt, fb = _tli_case(rng, Vd, Vt, K)
    d2t, t2d = otli.build_maps(inter, tgt, Vd, Vt, fb)
    # the draft distribution: softmax over the constrained (dense) draft logits
    pruned = (rng.standard_normal((3, K)) * 2).astype(np.float32)
    dense = otli.constrain_logits(pruned, inter, Vd)
    q_dense = torch.softmax(torch.from_numpy(dense.astype(np.float64)), 1).numpy().astype(np.float32)
    return inter, tgt, d2t, t2d, q_dense, Vt


def test_tli_q_scatter_carries_the_draft_distribution_into_target_ids():
    """A non-identity pairing: the scattered row is the draft distribution
    expressed in target ids (via the maps, which are pinned on their own), and
    it keeps the row's mass."""
    inter, tgt, d2t, t2d, q_dense, Vt = _q_scatter_case()
    q_target = otli.q_scatter(q_dense[:, inter], tgt, Vt)
    assert _q_target_semantics_hold(q_target, q_dense, d2t, t2d)
    for r in range(q_dense.shape[0]):
        assert sorted(q_target[r][q_target[r] != 0].tolist()) == sorted(q_dense[r][q_dense[r] != 0].tolist())
        assert abs(q_target[r].astype(np.float64).sum() - 1.0) < 1e-6


@pytest.mark.parametrize("plant", ["keyed_by_draft_ids", "keyed_by_column_through_d2t"])
def test_tli_q_scatter_planted_keys_are_caught(monkeypatch, plant):
    """Two plausible mistakes planted in the oracle's scatter -- keying it by
    the draft ids, or treating the column index as a draft id -- break the
    target-id semantics."""
    inter, tgt, d2t, t2d, q_dense, Vt = _q_scatter_case()
    orig = otli.q_scatter
    if plant == "keyed_by_draft_ids":
        monkeypatch.setattr(otli, "q_scatter", lambda q, ids, V: orig(q, np.asarray(inter) % V, V))
    else:
        cols = d2t[np.arange(len(inter))]
        monkeypatch.setattr(otli, "q_scatter", lambda q, ids, V: orig(q[:, cols >= 0], cols[cols >= 0], V))
    q_target = otli.q_scatter(q_dense[:, inter], tgt, Vt)
    assert not _q_target_semantics_hold(q_target, q_dense, d2t, t2d)


def test_tli_validator_follows_the_pages_rules():
    """The PR's validation block: topk == 1 and num_draft_tokens ==
    num_steps + 1.  Its benchmark shape (topk 1, 5 draft tokens, so 4 steps)
    passes; a tree (topk 8) and mismatched chain lengths are refused."""
    otli.check_tli_shape(1, 4, 5)
    otli.check_tli_shape(1, 1, 2)
    for k, S, N in [(8, 5, 64), (2, 4, 5), (1, 4, 4), (1, 4, 6), (1, 0, 1), (0, 4, 5)]:
        with pytest.raises(ValueError):
            otli.check_tli_shape(k, S, N)
