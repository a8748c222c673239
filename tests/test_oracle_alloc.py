"""Pins of the oracle's KV allocation: the pages' slot count for a draft
(batch x topk x steps at once), the duplicated partial page of the page > 1,
topk > 1 layout, the topk = 1 extend of a request's own chain, the
rollback, and conservation of units across a whole speculative step with
the oracle's compaction."""
import numpy as np
import pytest

from oracle import alloc as oal
from oracle import compact as ocmp


def test_page1_draft_takes_batch_x_topk_x_steps_slots_and_rolls_back():
    a = oal.KVAllocator(1000)
    before = (a.free_ids.copy(), a.top, a.pushes)
    bk = a.backup()
    B, topk, S = 5, 4, 3
    pages, loc, _, _ = oal.alloc_branches(a, np.zeros((B, 1), np.int32), np.array([7, 0, 13, 2, 9]), topk, S, 1)
    assert a.top == 1000 - B * topk * S
    assert len(set(loc.ravel().tolist())) == B * topk * S and (loc >= 0).all()
    assert np.array_equal(pages, loc)                      # P = 1: a page is a slot
    assert loc.ravel().tolist() == list(range(B * topk * S))   # fresh stack: ascending, (b, j, i) order
    a.restore(bk)
    assert a.error == 0 and a.top == before[1] and np.array_equal(a.free_ids, before[0])


def test_duplicated_partial_page_layout():
    """P = 4, prefix 6 (one full page + 2 tokens), topk 3, 3 steps: every
    branch gets ceil((2 + 3) / 4) = 2 pages; its first two slots hold copies
    of the prefix's two partial-page rows and its draft steps follow."""
    P, L, topk, S = 4, 6, 3, 3
    a = oal.KVAllocator(64)
    table = np.full((1, 8), -1, np.int32)
    table[0, :2] = a.pop(2)                                 # the prefix's pages (0, 1)
    rng = np.random.default_rng(0)
    layers = 2
    kp = [rng.integers(0, 60000, size=(64 * P, 2, 8)).astype(np.uint16) for _ in range(layers)]
    vp = [rng.integers(0, 60000, size=(64 * P, 2, 8)).astype(np.uint16) for _ in range(layers)]
    pages, loc, kp2, vp2 = oal.alloc_branches(a, table, np.array([L]), topk, S, P, kp, vp)
    assert pages[0].tolist() == [[2, 3], [4, 5], [6, 7]]
    partial = table[0, 1] * P                              # slots of the prefix's positions 4, 5
    for j in range(topk):
        first = pages[0, j, 0] * P
        for pool, orig in zip(kp2 + vp2, kp + vp):
            assert np.array_equal(pool[first:first + 2], orig[partial:partial + 2])
        assert loc[0, j].tolist() == [first + 2, first + 3, pages[0, j, 1] * P]
    # nothing else moved
    for pool, orig in zip(kp2 + vp2, kp + vp):
        moved = np.zeros(len(orig), bool)
        for j in range(topk):
            moved[pages[0, j, 0] * P:pages[0, j, 0] * P + 2] = True
        assert np.array_equal(pool[~moved], orig[~moved])


def test_page_aligned_prefix_needs_no_copy():
    P = 8
    a = oal.KVAllocator(40)
    table = np.full((2, 6), -1, np.int32)
    table[0, :2] = a.pop(2)
    table[1, :1] = a.pop(1)
    kp = [np.arange(40 * P * 4, dtype=np.uint16).reshape(40 * P, 1, 4)]
    pages, loc, kp2, _ = oal.alloc_branches(a, table, np.array([16, 8]), 2, 9, P, kp, [])
    assert np.array_equal(kp2[0], kp[0])
    assert (pages >= 0).all() and pages.shape[2] == 2      # r = 0: 9 steps take 2 pages, the most any r needs
    assert loc[0, 0].tolist() == [pages[0, 0, 0] * P + i for i in range(8)] + [pages[0, 0, 1] * P]


def test_topk1_extend_continues_the_partial_page():
    P = 4
    a = oal.KVAllocator(32)
    table = np.full((2, 6), -1, np.int32)
    table[0, :2] = a.pop(2)                                 # length 6: pages 0, 1 (page 1 half full)
    table[1, :1] = a.pop(1)                                 # length 4: page 2 full
    t2, loc = oal.alloc_extend(a, table, np.array([6, 4]), 5, P)
    # request 0: positions 6..10 finish page 1 and need one new page; request 1:
    # positions 4..8 need two new pages
    assert t2[0, :4].tolist() == [0, 1, 3, -1] and t2[1, :4].tolist() == [2, 4, 5, -1]
    assert loc[0].tolist() == [1 * P + 2, 1 * P + 3, 3 * P, 3 * P + 1, 3 * P + 2]
    assert loc[1].tolist() == [4 * P, 4 * P + 1, 4 * P + 2, 4 * P + 3, 5 * P]
    a1 = oal.KVAllocator(50)
    tab = np.full((1, 20), -1, np.int32)
    tab[0, :3] = a1.pop(3)
    t3, loc1 = oal.alloc_extend(a1, tab, np.array([3]), 4, 1)  # P = 1: the table is a slot map
    assert t3[0, 3:7].tolist() == [3, 4, 5, 6] == loc1[0].tolist()


def test_all_or_nothing_and_rollback_rules():
    a = oal.KVAllocator(10)
    table = np.full((2, 4), -1, np.int32)
    t2, loc = oal.alloc_extend(a, table, np.array([0, 0]), 6, 1)    # needs 12 > 10
    assert a.error & 1 and a.top == 10 and (loc == -1).all() and np.array_equal(t2, table)
    a.error = 0
    t2, loc = oal.alloc_extend(a, np.full((1, 4), -1, np.int32), np.array([2]), 3, 1)   # row overflow
    assert a.error & 1 and a.top == 10
    a = oal.KVAllocator(10)
    bk = a.backup()
    a.pop(4)
    a.push([2])
    a.restore(bk)
    assert a.error & 2 and a.top == 7
    a.push(list(range(5)))                                  # would exceed the capacity
    assert a.error & 4 and a.top == 7


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_units_are_conserved_over_speculative_steps(seed):
    """Several rounds of: draft branches (P = 1) then rollback; verify tree
    extend; compaction of a random accepted path; release of the freed slots.
    Every slot is always either free or in a request's slot map, never both,
    and the free stack has no duplicates."""
    rng = np.random.default_rng(seed)
    B, N, S, topk, cap = 6, 9, 3, 3, 400
    a = oal.KVAllocator(cap)
    max_pos = 200
    table = np.full((B, max_pos), -1, np.int32)
    seq = rng.integers(1, 20, size=B).astype(np.int32)
    for b in range(B):
        table[b, :seq[b]] = a.pop(int(seq[b]))
    for _ in range(4):
        bk = a.backup()
        oal.alloc_branches(a, table, seq, topk, S, 1)
        a.restore(bk)
        table, _ = oal.alloc_extend(a, table, seq, N, 1)
        acc = rng.integers(0, S + 1, size=B).astype(np.int32)
        path = np.full((B, S + 1), -1, np.int32)
        for b in range(B):
            path[b, :acc[b] + 1] = np.sort(np.concatenate([[0], rng.choice(np.arange(1, N), acc[b], replace=False)]))
        table, _, _, new_len, freed = ocmp.compact_kv(table, [], [], seq, acc, path, N, 1)
        a.push(freed)
        seq = new_len
        assert a.error == 0
        free = a.free_ids[:a.top].tolist()
        used = [int(x) for b in range(B) for x in table[b, :seq[b]]]
        assert len(set(free)) == len(free) and len(set(used)) == len(used)
        assert not set(free) & set(used) and len(free) + len(used) == cap
        assert (table[np.arange(max_pos)[None, :] >= seq[:, None]] == -1).all()
