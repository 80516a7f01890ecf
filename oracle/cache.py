"""Appending a verify block's K/V rows to the stores, committing the accepted ones.
TEST INFRASTRUCTURE ONLY.

Definition (lucebox post "Laguna XS 2.1 33B on a RTX 3090: 296 tok/s peak, 152 tok/s at 256K
context"):

* The verify block is one batched forward over the drafted tokens ("The model, fast MoE with a
  drafter in the box"), so its own K/V rows (positions ctx .. ctx+n-1) are in the stores when
  its attention runs, and the tokens it keeps are exactly those plain greedy decoding by the
  target would have produced (same section: the verification is greedy-exact).
* Window layers keep a ring indexed by position, slot = pos mod 2048 ("3. Ring caches for the
  sliding-window layers"): row of position p is written at ring slot p mod R.
* Full-attention layers keep a pool of 64-token chunks located through a page table ("Three
  optimizations", item 1): position p lives in slot table[p // 64] at offset p % 64.

Readings (the pages are silent on them; the plain ones): a rejected row is left where it is
and is overwritten by the next block, which writes the same positions before its attention
reads them; a chunk of the pool is given a slot when a block first writes one of its
positions, and a chunk the block started that keeps no committed position gives its slot
back.  Which free slot is handed out is a policy, not part of the method; ``PagerModel``
states the one the library uses (a stack that starts as 0, 1, 2, ...; a block's unused
chunks are returned last chunk first, so the earliest is handed out first again).

Host paging (same post, "Three optimizations", item 1: only part of the context stays in the
GPU pool, 64-token chunks that are not needed move to host memory without any change to their
bits, and which chunks stay is a scoring question outside this path).  A host chunk store holds one entry per logical chunk, laid out like
a pool slot; paging a chunk out copies its slot to the chunk's host entry and frees the slot,
paging it in copies the entry into a free slot.  Attention of a block over the resident subset
attends exactly the keys of the chunks that have a slot, at their own positions.

Readings: only whole committed chunks (every position below the committed length, and not the
chunk the next block writes into) can be paged out; a paged-out chunk's table entry is -2; the
slots freed by a page-out return to the same free stack as the pager's, in the order given.

Stores: K ``[slot][Hkv][64][D]``, V dimension-major ``[slot][Hkv][D][64]`` (as in
``attention``).  Arrays are copied, never modified in place.
"""
from __future__ import annotations

import numpy as np

from .attention import attend_rows, to_f64

CHUNK = 64
PAGED_OUT = -2


def append_ring(k_ring, v_ring, k_new, v_new, pos_first: int):
    """Rows k_new, v_new [n][Hkv][D] (positions pos_first ..) written at slot pos mod R (lucebox
    post, "3. Ring caches for the sliding-window layers")."""
    k = np.array(k_ring, copy=True)
    v = np.array(v_ring, copy=True)
    ring = k.shape[0] * CHUNK
    for i in range(k_new.shape[0]):
        s = (pos_first + i) % ring
        for g in range(k_new.shape[1]):
            k[s // CHUNK, g, s % CHUNK, :] = k_new[i, g, :]
            v[s // CHUNK, g, :, s % CHUNK] = v_new[i, g, :]
    return k, v


def append_paged(k_pool, v_pool, table, k_new, v_new, pos_first: int):
    """Rows written at slot table[pos // 64], offset pos % 64 (the table already holds the
    slots of the chunks the rows fall in; lucebox post, "Three optimizations", item 1)."""
    k = np.array(k_pool, copy=True)
    v = np.array(v_pool, copy=True)
    for i in range(k_new.shape[0]):
        p = pos_first + i
        slot = table[p // CHUNK]
        for g in range(k_new.shape[1]):
            k[slot, g, p % CHUNK, :] = k_new[i, g, :]
            v[slot, g, :, p % CHUNK] = v_new[i, g, :]
    return k, v


def page_out(k_pool, v_pool, slots, chunk_ids, k_host, v_host):
    """Host entries chunk_ids[i] <- pool slot slots[i] (K and V), bit for bit (lucebox post,
    "Three optimizations", item 1: chunks move between the pool and host memory).  Returns the new host stores."""
    kh = np.array(k_host, copy=True)
    vh = np.array(v_host, copy=True)
    for s, c in zip(slots, chunk_ids):
        kh[c] = k_pool[s]
        vh[c] = v_pool[s]
    return kh, vh


def page_in(k_host, v_host, chunk_ids, slots, k_pool, v_pool):
    """Pool slots slots[i] <- host entries chunk_ids[i] (K and V), bit for bit (same passage).
    Returns the new pool."""
    kp = np.array(k_pool, copy=True)
    vp = np.array(v_pool, copy=True)
    for c, s in zip(chunk_ids, slots):
        kp[s] = k_host[c]
        vp[s] = v_host[c]
    return kp, vp


def attention_resident(q, k_pool, v_pool, chunk_ids, slots, ctx_len, scale=None, dtype="bf16"):
    """Attention of the block over the resident chunks only (lucebox post, "Three optimizations",
    item 1: only part of the context stays in the pool): the keys are positions
    c*64 .. c*64+63 (below ctx_len) of every listed chunk c, read from pool slot slots[i]; query
    i sits at ctx_len - q_len + i and sees the listed keys at or before its own position."""
    qf = to_f64(q, dtype)
    q_len, _, d = qf.shape
    key_pos, key_slot, key_off = [], [], []
    for c, s in zip(chunk_ids, slots):
        for t in range(CHUNK):
            if c * CHUNK + t < ctx_len:
                key_pos.append(c * CHUNK + t)
                key_slot.append(s)
                key_off.append(t)
    key_pos = np.array(key_pos, dtype=np.int64)
    ks, ko = np.array(key_slot, dtype=np.int64), np.array(key_off, dtype=np.int64)
    kp, vp = np.asarray(k_pool), np.asarray(v_pool)
    sc = 1.0 / np.sqrt(d) if not scale else float(scale)
    return attend_rows(qf, lambda g: to_f64(kp[ks, g, ko, :], dtype),
                       lambda g: to_f64(vp[ks, g, :, ko], dtype), key_pos,
                       ctx_len - q_len + np.arange(q_len), 0, sc, kp.shape[1])


class PagerModel:
    """Slot bookkeeping of one sequence's pool chunks: committed length, table, free stack
    (lucebox post, "Three optimizations", item 1 for the chunk pool; "The model, fast MoE with a
    drafter in the box" for committing only the target's own tokens; the allocation policy is
    a reading, stated above)."""

    def __init__(self, n_slots: int, n_table: int):
        self.table = [-1] * n_table
        self.free = list(range(n_slots - 1, -1, -1))   # pop() hands out 0, 1, 2, ...
        self.ctx = 0
        self.pending = None                             # (n, first chunk, chunks started)

    def reserve(self, n: int):
        """Slots for the chunks positions ctx .. ctx+n-1 start: (first_chunk, slots)."""
        if self.pending is not None or not 1 <= n <= 1024:
            raise ValueError("reserve")
        first = -(-self.ctx // CHUNK)                  # first chunk without a position yet
        end = -(-(self.ctx + n) // CHUNK)
        if end > len(self.table) or end - first > len(self.free):
            raise MemoryError("pool or table exhausted")
        slots = []
        for c in range(first, end):
            s = self.free.pop()
            self.table[c] = s
            slots.append(s)
        self.pending = (n, first, end - first)
        return first, slots

    def commit(self, n_keep: int):
        """The block's first n_keep rows are committed; its chunks past them are freed."""
        if self.pending is None or not 0 <= n_keep <= self.pending[0]:
            raise ValueError("commit")
        _, first, k = self.pending
        self.ctx += n_keep
        keep = -(-self.ctx // CHUNK)
        for c in range(first + k - 1, first - 1, -1):
            if c < keep:
                break
            self.free.append(self.table[c])
            self.table[c] = -1
        self.pending = None

    def evict(self, chunk_ids):
        """Page out whole committed chunks: their slots (returned, in the order given) go back
        to the free stack and their table entries become PAGED_OUT.  All or nothing."""
        full = self.ctx // CHUNK                        # chunks whose 64 positions are committed
        ids = list(chunk_ids)
        if len(set(ids)) != len(ids) or any(not 0 <= c < full or self.table[c] < 0 for c in ids):
            raise ValueError("evict")
        slots = [self.table[c] for c in ids]
        for c in ids:
            self.free.append(self.table[c])
            self.table[c] = PAGED_OUT
        return slots

    def restore(self, chunk_ids):
        """Page chunks back in: each gets the next free slot (returned, in the order given)."""
        ids = list(chunk_ids)
        if len(set(ids)) != len(ids) or any(not 0 <= c < len(self.table) or
                                            self.table[c] != PAGED_OUT for c in ids):
            raise ValueError("restore")
        if len(ids) > len(self.free):
            raise MemoryError("pool exhausted")
        slots = []
        for c in ids:
            s = self.free.pop()
            self.table[c] = s
            slots.append(s)
        return slots

    def resident(self):
        """(chunk ids, slots) of every chunk that has a slot, in increasing chunk order."""
        ids = [c for c, s in enumerate(self.table) if s >= 0]
        return ids, [self.table[c] for c in ids]
