"""Greedy acceptance of a drafted block.  TEST INFRASTRUCTURE ONLY.

The target scores k drafted tokens in one forward and yields k+1 logit rows: row r
is the target's distribution for the token after the committed prefix plus
drafts 0..r-1 (row k follows the whole draft).  Greedy acceptance commits the
longest drafted prefix on which the target's argmax agrees, then the target's own
token at the first disagreement (or after the last draft):

    t_r = min { v : L[r][v] = max_u L[r][u] }           r = 0..k (first maximum)
    a   = min ({ r < k : t_r != prop[r] } U { k })
    committed = prop[0..a) ++ [t_a]                      a + 1 tokens

If row r is the target's distribution given the committed prefix and prop[0..r),
then committed equals a+1 steps of plain greedy decoding, so the output is exactly
the target's own (lucebox post "Laguna XS 2.1 33B on a RTX 3090: 296 tok/s peak,
152 tok/s at 256K context", "The model, fast MoE with a drafter in the box": the
proposals are verified in one batched forward and what is kept equals greedy decoding
by the target; "TL;DR": the decode is verify-exact).

The argmax compares float32 values as float32 (the logits' own precision); -0.0 and
+0.0 compare equal, so the lower index wins.  Inputs must be finite.
"""
from __future__ import annotations

import numpy as np


def first_argmax(row) -> int:
    """Index of the first maximum of a float32 row, by a plain left-to-right scan."""
    row = np.asarray(row, dtype=np.float32)
    best = 0
    for v in range(1, row.shape[0]):
        if row[v] > row[best]:
            best = v
    return best


def greedy_accept(logits, proposals, scan=False):
    """Returns (accept_len a, committed [a+1] int32, row_argmax [k+1] int32).

    ``scan=True`` uses the explicit left-to-right scan for the argmax (slow, small
    inputs); otherwise ``numpy.argmax`` on the float32 rows, which also returns the
    first maximum."""
    L = np.asarray(logits, dtype=np.float32)
    prop = np.asarray(proposals, dtype=np.int64)
    k = prop.shape[0]
    if L.shape[0] != k + 1:
        raise ValueError("need k+1 logit rows for k proposals")
    if not np.all(np.isfinite(L)):
        raise ValueError("logits must be finite")
    t = np.array([first_argmax(L[r]) for r in range(k + 1)] if scan else np.argmax(L, axis=1),
                 dtype=np.int64)
    a = k
    for r in range(k):
        if t[r] != prop[r]:
            a = r
            break
    committed = np.concatenate([prop[:a], t[a:a + 1]]).astype(np.int32)
    return a, committed, t.astype(np.int32)
