"""Oracle: KV slot / page allocation around a speculative step.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Follows "EAGLE speculative decoding in four parts", "Drafting, verification
and slots": with page size 1 the draft reserves num_seqs * topk * num_steps
slots at once and backs up the allocator's state, which is rolled back after
the step; with a larger page size and topk = 1 each request extends its own
sequence by num_steps tokens, and with topk > 1 the last partial page is
duplicated, so that every branch holds a copy of the prefix's partial page
followed by its own draft tokens (the page-table layout drawn there as
"| prefix pages | partial + branch 0 | partial + branch 1 | ...").
"Design trade-offs": allocate first, roll back after.  "[SGLang] Multi-Layer
EAGLE", section 6: draft and target share one allocator.

Readings where the pages leave a step open:
* Units are slots when the page size P is 1 and pages when P > 1.  The free
  units form a stack: free_ids[0 .. top) with free_ids[top - 1] handed out
  first; a release pushes ids in the order given.  A fresh allocator holds
  0 .. capacity-1 so that they come out in ascending order.
* The state is (top, pushes): a backup records both; a restore is allowed
  only if nothing was pushed since the backup (then the units popped since
  are exactly those above the backed-up top, still in place), and sets top
  back.  Anything else is an error and changes nothing.
* All requests are served in batch order, all-or-nothing: if the batch needs
  more units than are free, or a request's table row would overflow, nothing
  is allocated and an error is recorded.
* extend (verify tree, topk = 1 draft): request b of length L = seq_len[b]
  takes positions L .. L+n-1 of its own chain.  P = 1: one slot per
  position, table[b][L+i] = the slot.  P > 1: the partial last page (if any)
  is continued, the new pages ceil(L/P) .. ceil((L+n)/P)-1 are taken in
  order.  out_loc[b][i] = slot of position L+i (page * P + offset).
* branches (topk > 1 draft, or P = 1): with r = L mod P, branch j of request
  b takes ceil((r + S) / P) pages of its own (requests, then branches, then
  pages in order); its first r slots receive a copy of the K and V rows of
  the prefix's partial page (every layer), and draft step i of the branch is
  at slot branch_pages[b][j][(r+i) // P] * P + (r+i) mod P.  With P = 1 this
  is one slot per (request, branch, step), B*topk*S in all.
"""
from __future__ import annotations

import numpy as np


class KVAllocator:
    """Device-layout twin: free_ids [capacity] and state = (top, pushes, error)."""

    def __init__(self, capacity: int):
        if capacity < 0:
            raise ValueError("capacity must be non-negative")
        self.capacity = capacity
        self.free_ids = np.arange(capacity - 1, -1, -1, dtype=np.int32)   # pops give 0, 1, 2, ...
        self.top = capacity
        self.pushes = 0
        self.error = 0

    def state(self):
        return np.array([self.top, self.pushes, self.error, 0], np.int32)

    def pop(self, n: int):
        if n > self.top:
            raise ValueError("not enough free units")
        out = [int(self.free_ids[self.top - 1 - i]) for i in range(n)]
        self.top -= n
        return out

    def push(self, ids):
        ids = [int(x) for x in ids]
        if self.top + len(ids) > self.capacity:
            self.error |= 4
            return
        for i, x in enumerate(ids):
            self.free_ids[self.top + i] = x
        self.top += len(ids)
        self.pushes += 1

    def backup(self):
        return (self.top, self.pushes)

    def restore(self, backup):
        top, pushes = backup
        if pushes != self.pushes or top < self.top or top > self.capacity:
            self.error |= 2
            return
        self.top = top


def _extend_need(L: int, n: int, P: int) -> int:
    if P == 1:
        return n
    return -(-(L + n) // P) - (-(-L // P))


def alloc_extend(alloc: KVAllocator, page_table, seq_len, n: int, P: int):
    """Positions L .. L+n-1 of every request's own chain.  Returns
    (page_table', out_loc [B, n]); on failure the error flag is set and the
    inputs come back unchanged (out_loc all -1)."""
    table = np.array(page_table, dtype=np.int32, copy=True)
    B, max_pages = table.shape
    out = np.full((B, n), -1, np.int32)
    need = [_extend_need(int(seq_len[b]), n, P) for b in range(B)]
    fits = all(-(-(int(seq_len[b]) + n) // P) <= max_pages for b in range(B))
    if not fits or sum(need) > alloc.top:
        alloc.error |= 1
        return table, out
    for b in range(B):
        L = int(seq_len[b])
        ids = alloc.pop(need[b])
        if P == 1:
            for i in range(n):
                table[b, L + i] = ids[i]
        else:
            first = -(-L // P)
            for t, pid in enumerate(ids):
                table[b, first + t] = pid
        for i in range(n):
            pos = L + i
            out[b, i] = table[b, pos // P] * P + pos % P
    return table, out


def alloc_branches(alloc: KVAllocator, page_table, seq_len, topk: int, S: int, P: int, k_pools=(), v_pools=()):
    """Per-branch draft regions.  Returns (branch_pages [B, topk, maxpb] (-1
    padded), out_loc [B, topk, S], k_pools', v_pools').  The pools (lists of
    [slots, Hkv, D] arrays, one per layer; P > 1 only) get the partial-page
    copies."""
    table = np.asarray(page_table, dtype=np.int32)
    B = table.shape[0]
    maxpb = -(-(P - 1 + S) // P) if P > 1 else S
    pages = np.full((B, topk, maxpb), -1, np.int32)
    out = np.full((B, topk, S), -1, np.int32)
    kp = [np.array(x, copy=True) for x in k_pools]
    vp = [np.array(x, copy=True) for x in v_pools]
    per = [-(-((int(seq_len[b]) % P) + S) // P) for b in range(B)]
    if sum(per) * topk > alloc.top:
        alloc.error |= 1
        return pages, out, kp, vp
    for b in range(B):
        L = int(seq_len[b])
        r = L % P
        for j in range(topk):
            ids = alloc.pop(per[b])
            pages[b, j, :len(ids)] = ids
            for i in range(S):
                out[b, j, i] = ids[(r + i) // P] * P + (r + i) % P
            src = int(table[b, L // P]) * P if r else 0
            for t in range(r):
                for pool in kp + vp:
                    pool[ids[0] * P + t] = pool[src + t]
    return pages, out, kp, vp
