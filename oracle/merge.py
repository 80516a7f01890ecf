"""Split-K partials and their log-sum-exp merge, float64.  TEST INFRASTRUCTURE ONLY.

Attention over a key set J that is the disjoint union of parts J_1 .. J_S can be
computed part by part.  Each part gives a normalised output O_s and lse_s over its
own keys (a query with no visible key in the part gives lse_s = -inf and carries no
weight).  The whole is

    M = max_s lse_s,   w_s = exp(lse_s - M),
    O = sum_s w_s O_s / sum_s w_s,   lse = M + ln sum_s w_s

which is the plain softmax over J regrouped: exp(lse_s) is the part's sum of
exp(score), so w_s / sum w_s is the part's share of the total weight.  Long
contexts are split this way across chunk ranges and merged.
"""
from __future__ import annotations

import numpy as np

from .attention import attend_rows


def attention_partial(q, k_of_head, v_of_head, key_pos, q_pos, window, scale, n_kv_heads):
    """Attention restricted to the listed keys (one part of a split of the key range; the pages
    describe no split, so the part boundaries are the caller's)."""
    return attend_rows(q, k_of_head, v_of_head, key_pos, q_pos, window, scale, n_kv_heads)


def lse_merge(parts):
    """Merge ``[(O_s, lse_s), ...]`` over disjoint key parts (shapes [..., D] and [...]): the
    regrouping of one softmax over the union stated above, exact up to rounding."""
    lses = np.stack([np.asarray(l, dtype=np.float64) for _, l in parts])      # [S, ...]
    outs = np.stack([np.asarray(o, dtype=np.float64) for o, _ in parts])      # [S, ..., D]
    M = lses.max(axis=0)
    has = np.isfinite(M)
    Mz = np.where(has, M, 0.0)
    w = np.where(np.isfinite(lses), np.exp(lses - Mz[None]), 0.0)             # [S, ...]
    tot = w.sum(axis=0)
    out = np.zeros(outs.shape[1:], dtype=np.float64)
    num = (w[..., None] * outs).sum(axis=0)
    out[has] = num[has] / tot[has][..., None]
    lse = np.full(M.shape, -np.inf)
    lse[has] = M[has] + np.log(tot[has])
    return out, lse
