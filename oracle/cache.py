"""Appending a verify block's K/V rows to the stores, committing the accepted ones.
TEST INFRASTRUCTURE ONLY.

Definition (lucebox post "Laguna XS 2.1 33B on a RTX 3090: 296 tok/s peak, 152 tok/s at 256K
context"):

* The verify block is one batched forward over the drafted tokens ("The model, fast MoE with a
  drafter in the box"), so its own K/V rows (positions ctx .. ctx+n-1) are in the stores when
  its attention runs, and only the tokens the target itself would emit are committed (same
  section, "commits only tokens the target itself would emit").
* Window layers keep a position ring, slot = pos mod 2048 ("3. Ring caches for the
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

Stores: K ``[slot][Hkv][64][D]``, V dimension-major ``[slot][Hkv][D][64]`` (as in
``attention``).  Arrays are copied, never modified in place.
"""
from __future__ import annotations

import numpy as np

CHUNK = 64


def append_ring(k_ring, v_ring, k_new, v_new, pos_first: int):
    """Rows k_new, v_new [n][Hkv][D] (positions pos_first ..) written at slot pos mod R."""
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
    slots of the chunks the rows fall in)."""
    k = np.array(k_pool, copy=True)
    v = np.array(v_pool, copy=True)
    for i in range(k_new.shape[0]):
        p = pos_first + i
        slot = table[p // CHUNK]
        for g in range(k_new.shape[1]):
            k[slot, g, p % CHUNK, :] = k_new[i, g, :]
            v[slot, g, :, p % CHUNK] = v_new[i, g, :]
    return k, v


class PagerModel:
    """Slot bookkeeping of one sequence's pool chunks: committed length, table, free stack."""

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
