"""Verify-block attention, float64, two-pass softmax.  TEST INFRASTRUCTURE ONLY.

Definition (every store layout):

    query i of the block sits at position p_i; q-head h reads KV head g = h // G,
    G = Hq / Hkv (grouped-query attention, contiguous groups).
    keys visible to query i:  0 <= j <= p_i                     (full causal)
                              max(0, p_i - W + 1) <= j <= p_i    (sliding window W: W keys
                                                                 including the query's own)
    s_j   = scale * <Q[i,h,:], K(j)[g,:]>
    m     = max_j s_j,  w_j = exp(s_j - m),  l = sum_j w_j
    O     = sum_j w_j V(j)[g,:] / l,   lse = m + ln l

The verify block is one batched forward over all proposals (lucebox post
"Laguna XS 2.1 33B on a RTX 3090: 296 tok/s peak, 152 tok/s at 256K context",
section "The model, fast MoE with a drafter in the box"), so query i sees the
block's earlier tokens and itself: it must equal single-token decoding with
context p_i + 1.  The window is the post's 512-token sliding window (same section
and "3. Ring caches for the sliding-window layers").

Where K(j), V(j) come from:

* contiguous rows ``K[j][g][:]``;
* the position ring (same post, "3. Ring caches for the sliding-window layers":
  slot = pos mod 2048): slot s = j mod R, stored as chunk slot s // 64 at offset s % 64;
* the paged pool of 64-token chunks (same post, "Three optimizations" item 1): logical
  chunk c = j // 64 lives in pool slot page_table[c], at offset j % 64.

Chunked stores hold K as ``[slot][Hkv][64][D]`` and V dimension-major as
``[slot][Hkv][D][64]`` (the layout the C interface states).
"""
from __future__ import annotations

import numpy as np

CHUNK = 64


def bf16_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) to float64, exactly: the bf16 bits are the high half of
    a float32."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def to_f64(x, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_to_f64(x)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if dtype == "f64":
        return np.asarray(x, dtype=np.float64)
    raise ValueError(dtype)


def key_bounds(p: int, window: int):
    """Inclusive range of key positions visible to a query at position ``p``: all earlier
    positions and its own, or the last ``window`` of them (lucebox post, "3. Ring caches for the
    sliding-window layers": the 512-token window; W keys including the query's own)."""
    lo = max(0, p - window + 1) if window > 0 else 0
    return lo, p


def attend_rows(q, k_of_head, v_of_head, key_pos, q_pos, window, scale, n_kv_heads):
    """Attention of the block over an explicit key list: the softmax definition above, for
    the one batched forward over the proposals (lucebox post, "The model, fast MoE with a
    drafter in the box").

    q          [q_len][Hq][D] float64
    k_of_head  callable g -> [n][D] float64: K(key_pos[j])[g] for every listed key
    v_of_head  callable g -> [n][D] float64
    key_pos    [n] int, the position of each listed key
    q_pos      [q_len] int, the position of each query
    Keys listed but not visible to a query (outside its causal/window range) get no
    weight.  Returns out [q_len][Hq][D], lse [q_len][Hq]; a query with no visible key
    gets out = 0, lse = -inf.
    """
    q = np.asarray(q, dtype=np.float64)
    q_len, hq, d = q.shape
    G = hq // n_kv_heads
    key_pos = np.asarray(key_pos, dtype=np.int64)
    q_pos = np.asarray(q_pos, dtype=np.int64)
    lo = np.array([key_bounds(int(p), window)[0] for p in q_pos], dtype=np.int64)
    visible = (key_pos[None, :] >= lo[:, None]) & (key_pos[None, :] <= q_pos[:, None])
    out = np.zeros((q_len, hq, d), dtype=np.float64)
    lse = np.full((q_len, hq), -np.inf, dtype=np.float64)
    for g in range(n_kv_heads):
        Kg = k_of_head(g)
        Vg = v_of_head(g)
        for h in range(g * G, (g + 1) * G):
            s = scale * (q[:, h, :] @ Kg.T)                  # [q_len][n]
            s = np.where(visible, s, -np.inf)
            m = s.max(axis=1) if s.shape[1] else np.full(q_len, -np.inf)
            has = np.isfinite(m)
            w = np.exp(s - np.where(has, m, 0.0)[:, None])   # masked keys: exp(-inf) = 0
            l = w.sum(axis=1)
            o = w @ Vg
            out[has, h, :] = o[has] / l[has, None]
            lse[has, h] = m[has] + np.log(l[has])
    return out, lse


def _scale(scale, d):
    return 1.0 / np.sqrt(d) if not scale else float(scale)


def attention_contiguous(q, k, v, ctx_len, window=0, scale=None, dtype="f64", q_len=None):
    """Contiguous rows ``k, v [ctx][Hkv][D]``; query i at position ctx_len - q_len + i (the
    block counted in the context, as one batched forward over the proposals: lucebox post, "The
    model, fast MoE with a drafter in the box")."""
    qf = to_f64(q, dtype)
    q_len = qf.shape[0] if q_len is None else q_len
    kf = to_f64(np.asarray(k)[:ctx_len], dtype)
    vf = to_f64(np.asarray(v)[:ctx_len], dtype)
    hkv = kf.shape[1]
    q_pos = ctx_len - q_len + np.arange(q_len)
    if q_pos[0] < 0:
        raise ValueError("the block is longer than the context")
    key_pos = np.arange(ctx_len)
    return attend_rows(qf, lambda g: kf[:, g, :], lambda g: vf[:, g, :], key_pos, q_pos, window,
                       _scale(scale, qf.shape[2]), hkv)


def gather_ring(k_ring, v_ring, positions, ring_size, chunk=CHUNK):
    """K(j), V(j) for positions ``j`` read from the ring at slot j mod ring_size (lucebox post,
    "3. Ring caches for the sliding-window layers": slot = pos mod 2048).

    Returns two callables g -> [n][D] (raw element type, not converted)."""
    positions = np.asarray(positions, dtype=np.int64)
    slot = positions % ring_size
    cs, off = slot // chunk, slot % chunk
    return (lambda g: np.asarray(k_ring)[cs, g, off, :],
            lambda g: np.asarray(v_ring)[cs, g, :, off])


def attention_ring(q, k_ring, v_ring, pos0, ring_head, ring_size, window, scale=None,
                   dtype="bf16", chunk=CHUNK):
    """Sliding-window verify attention over a position ring (lucebox post, "3. Ring caches for
    the sliding-window layers").

    Query i sits at pos0 + i; the ring holds the last ``ring_size`` positions up to
    pos0 + q_len - 1 (the block's own rows included).  Raises if a visible position
    is no longer resident (the ring is too small for window + block) or if
    ``ring_head`` is not the slot of ``pos0``.
    """
    qf = to_f64(q, dtype)
    q_len = qf.shape[0]
    if ring_head != pos0 % ring_size:
        raise ValueError("ring_head must be the slot of the block's first query")
    if window <= 0:
        raise ValueError("ring attention needs a window")
    q_pos = pos0 + np.arange(q_len)
    lo = key_bounds(int(q_pos[0]), window)[0]
    hi = int(q_pos[-1])
    resident_lo = max(0, hi - ring_size + 1)
    if lo < resident_lo:
        raise ValueError("a visible position has been overwritten in the ring")
    key_pos = np.arange(lo, hi + 1)
    kg, vg = gather_ring(k_ring, v_ring, key_pos, ring_size, chunk)
    return attend_rows(qf, lambda g: to_f64(kg(g), dtype), lambda g: to_f64(vg(g), dtype),
                       key_pos, q_pos, window, _scale(scale, qf.shape[2]), np.asarray(k_ring).shape[1])


def gather_paged(k_pool, v_pool, page_table, positions, chunk=CHUNK):
    """K(j), V(j) for positions ``j`` read from pool slot page_table[j // chunk] at j % chunk
    (lucebox post, "Three optimizations", item 1: the pool of 64-token chunks)."""
    positions = np.asarray(positions, dtype=np.int64)
    pt = np.asarray(page_table, dtype=np.int64)
    slot = pt[positions // chunk]
    off = positions % chunk
    return (lambda g: np.asarray(k_pool)[slot, g, off, :],
            lambda g: np.asarray(v_pool)[slot, g, :, off])


def attention_paged(q, k_pool, v_pool, page_table, ctx_len, scale=None, dtype="bf16",
                    chunk=CHUNK, window=0):
    """Full-attention (or windowed) verify attention over the paged pool (lucebox post,
    "Three optimizations", item 1).  Keys are positions 0 .. ctx_len-1; query i sits at
    ctx_len - q_len + i."""
    qf = to_f64(q, dtype)
    q_len = qf.shape[0]
    n_chunks = -(-ctx_len // chunk)
    pt = np.asarray(page_table)
    if len(pt) < n_chunks:
        raise ValueError("page table shorter than the context")
    n_slots = np.asarray(k_pool).shape[0]
    if n_chunks and (pt[:n_chunks].min() < 0 or pt[:n_chunks].max() >= n_slots):
        raise ValueError("page table entry outside the pool")
    q_pos = ctx_len - q_len + np.arange(q_len)
    lo = key_bounds(int(q_pos[0]), window)[0]
    key_pos = np.arange(lo, ctx_len)
    kg, vg = gather_paged(k_pool, v_pool, pt, key_pos, chunk)
    return attend_rows(qf, lambda g: to_f64(kg(g), dtype), lambda g: to_f64(vg(g), dtype),
                       key_pos, q_pos, window, _scale(scale, qf.shape[2]), np.asarray(k_pool).shape[1])
