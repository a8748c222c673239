"""Oracle: the index preparation of the draft extend that follows a verify step.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Follows "EAGLE speculative decoding in four parts", "Self-test" answer 1:
after verification the draft model runs one extend over the accepted tokens
to prepare the next round; zero-to-sglang ch.10, section 3.1: the worker's
step is draft, then verify, then the draft-side extend that readies the next
round's input; sglang PR #22883 ("Modifications", the hooks table): under TLI
the accepted tokens are mapped target -> draft for that extend and the
target-vocabulary ids are kept for everything else.

Readings where the pages leave a step open:
* The extend runs over the committed tokens of each request (the accepted
  draft tokens and the correction or bonus token, as the accept walk returns
  them), requests in batch order, packed without gaps: request b's rows start
  at extend_start[b] = the sum of commit_len over the requests before it.
* Committed token j of request b was chosen at tree node accept_path[b, j]
  (the walk commits one token per visited node, root first).  Its position is
  prefix_len[b] + 1 + j (the root sits at prefix_len[b], node path[d] at
  prefix_len[b] + d), and the target hidden state paired with it is the
  verify output row of the node that chose it: b * N + accept_path[b, j].
* last_index[b] is the row of the request's last committed token, whose draft
  output seeds the next round (-1 when the request committed nothing).
* seq_len[b] = prefix_len[b] + 1 + commit_len[b] is the request's length once
  the extend has run.
* TLI: input_ids = t2d[token] with the target -> draft map (ids outside the
  intersection already map to the caller's fallback there); without a map the
  ids pass through.
"""
from __future__ import annotations

import numpy as np


def draft_extend_prep(prefix_len, commit_len, commit_tokens, accept_path, N: int, t2d=None):
    """Returns dict(extend_start [B+1], input_ids, positions, hidden_index
    [total], last_index [B], seq_len [B]), all int32.

    prefix_len, commit_len: [B]; commit_tokens, accept_path: [B, S+1] as the
    accept walk writes them (-1 padded); t2d: None or [V_target] int32.
    """
    prefix_len = np.asarray(prefix_len, dtype=np.int64)
    commit_len = np.asarray(commit_len, dtype=np.int64)
    commit_tokens = np.asarray(commit_tokens)
    accept_path = np.asarray(accept_path)
    B = prefix_len.shape[0]
    start = [0]
    for b in range(B):
        c = int(commit_len[b])
        if c < 0 or c > commit_tokens.shape[1]:
            raise ValueError("commit_len out of range")
        start.append(start[-1] + c)
    total = start[-1]
    ids = np.empty(total, np.int32)
    pos = np.empty(total, np.int32)
    hid = np.empty(total, np.int32)
    last = np.full(B, -1, np.int32)
    seq = np.empty(B, np.int32)
    for b in range(B):
        c = int(commit_len[b])
        for j in range(c):
            row = start[b] + j
            tok = int(commit_tokens[b, j])
            node = int(accept_path[b, j])
            if tok < 0 or node < 0 or node >= N:
                raise ValueError("committed token %d of request %d has no token or node" % (j, b))
            ids[row] = tok if t2d is None else int(t2d[tok])
            pos[row] = int(prefix_len[b]) + 1 + j
            hid[row] = b * N + node
        if c > 0:
            last[b] = start[b] + c - 1
        seq[b] = int(prefix_len[b]) + 1 + c
    return dict(extend_start=np.asarray(start, np.int32), input_ids=ids, positions=pos, hidden_index=hid,
                last_index=last, seq_len=seq)
