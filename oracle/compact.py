"""Oracle: keep the accepted path's KV, free the rest of the tree's allocation.

Follows "EAGLE speculative decoding in four parts": slots for every candidate
are reserved before drafting and, after verification, only the slots on the
accepted path are kept and the rest freed; with a page size above 1 the last
page is copied too ("Self-test" answer 3; "Drafting, verification and slots";
"Design trade-offs", allocate first and roll back after).  zero-to-sglang
ch.10, section 5.2: after a rejection the cache is restored to the committed
path, and the correction or bonus token has no KV of its own yet.

Readings where the pages leave a step open:
* The tree of request b occupies logical positions L_b .. L_b+N-1 of the
  request's own chain (node j at L_b + j), starting inside the prefix's partial
  last page when the page size P > 1.
* After accepting path[0..a] (path[0] = 0 is the root), logical position
  L_b + d must hold the KV computed for node path[d]; new length L_b + a + 1.
* P = 1: the table is a slot map and compaction is an index remap:
  slot(L_b+d) <- old slot(L_b+path[d]); positions L_b+a+1 .. L_b+N-1 become -1
  and the old slots of the rejected nodes are freed in ascending node order.
* P > 1: K and V rows ([Hkv, D] per layer) are copied from position
  L_b+path[d] to L_b+d for d = 1..a where they differ, in increasing d (a later
  copy never reads what an earlier one wrote); logical pages from
  ceil(new_len / P) to (L_b+N-1) // P become -1 and are freed in page order.
* The freed list runs over requests in batch order.
"""
from __future__ import annotations

import numpy as np


def compact_kv(page_table, k_pools, v_pools, prefix_len, accept_len, accept_path, N: int,
               page: int):
    """Returns (page_table', k_pools', v_pools', new_len [B], freed [num_freed]).

    page_table [B, max_pages] int32 (P = 1: slot map); k_pools / v_pools: lists
    (one per layer) of [slots, Hkv, D] arrays (any dtype: bytes are moved).
    Inputs are not modified.
    """
    table = np.array(page_table, dtype=np.int32, copy=True)
    kp = [np.array(x, copy=True) for x in k_pools]
    vp = [np.array(x, copy=True) for x in v_pools]
    B = table.shape[0]
    new_len = np.zeros(B, np.int32)
    freed = []
    for b in range(B):
        L = int(prefix_len[b])
        a = int(accept_len[b])
        path = [int(x) for x in accept_path[b, :a + 1]]
        if path[0] != 0 or any(not (path[d - 1] < path[d] < N) for d in range(1, a + 1)):
            raise ValueError("accept path must start at the root and increase")
        new_len[b] = L + a + 1
        if page == 1:
            old = table[b, L:L + N].copy()
            for d in range(a + 1):
                table[b, L + d] = old[path[d]]
            table[b, L + a + 1:L + N] = -1
            kept = set(path)
            freed.extend(int(old[j]) for j in range(N) if j not in kept)
        else:
            def slot(pos):
                return int(page_table[b, pos // page]) * page + pos % page
            for d in range(1, a + 1):
                if path[d] != d:
                    src, dst = slot(L + path[d]), slot(L + d)
                    for pool in kp + vp:
                        pool[dst] = pool[src]
            first_free = -(-int(new_len[b]) // page)
            last_used = (L + N - 1) // page
            for pg in range(first_free, last_used + 1):
                freed.append(int(table[b, pg]))
                table[b, pg] = -1
    return table, kp, vp, new_len, np.asarray(freed, dtype=np.int32)
