"""CPU oracle for the draft-tree build and target-side verify path.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, obviously correct
CPU statement of what the path computes, written from the pages (numpy plus
Python ints; float64 wherever the pages leave the precision open).  It is
imported only by ``tests/``, by ``__graft_entry__.smoke()`` and by the
``cpu_baseline`` leg of ``bench.py``.  It shares no code with the HIP library
and never imports it; the only thing both sides share is the seeded input
generator in ``workloads``.

Modules and the passages they follow:

* ``topk``      -- per-row draft top-k (``fast_topk`` after the per-step softmax;
                   "[SGLang] Multi-Layer EAGLE", section 3, draft extend).
* ``softmax``   -- the processed distributions softmax(logits / T) that the
                   draft's top-k and the stochastic verify consume (same page
                   section 3; zero-to-sglang ch.10 section 5.1).
* ``tree``      -- frontier expansion with cumulative scores and the final tree
                   (``select_top_k_tokens`` / ``tree_info``, same page section 2;
                   ``build_eagle_tree`` in "EAGLE speculative decoding in four
                   parts", "Drafting, verification and slots" and "Exercises"),
                   plus the mask, positions and retrieve arrays.
* ``attention`` -- dense tree-masked attention in float64.
* ``accept``    -- greedy commit (zero-to-sglang ch.10, section 4.1) and
                   rejection sampling with the positive residual (section 5.1),
                   generalised to a tree.
* ``compact``   -- keep the accepted path's KV, free the rest ("Drafting,
                   verification and slots"; zero-to-sglang ch.10 section 5.2).
* ``tli``       -- Token-Level Intersection remaps, logit masking and the pruned
                   LM head (sglang PR #22883, "Modifications").
* ``alloc``     -- KV slot / page allocation with backup and rollback, and the
                   duplicated partial page of the page > 1, topk > 1 draft
                   ("EAGLE speculative decoding in four parts", "Drafting,
                   verification and slots", "Design trade-offs").
* ``extend``    -- index preparation of the draft extend after a verify step
                   ("EAGLE speculative decoding in four parts", "Self-test";
                   zero-to-sglang ch.10 section 3.1; PR #22883 hooks).

Every function that no test pins to something outside itself says
"parity unpinned" in its docstring.
"""
from . import topk, tree, attention, accept, compact, tli, extend, alloc  # noqa: F401

__all__ = ["topk", "tree", "attention", "accept", "compact", "tli", "extend", "alloc"]
