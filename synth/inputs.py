"""Primitive generators: seeded streams, bf16 rounding, chunked-store scatter,
planted logits.

Seed scheme: every tensor of every workload comes from its own numpy
``Generator`` seeded with ``SeedSequence([2026, workload_id, layer, stream])``;
K/V rows are drawn in blocks of 8192 rows, block b seeded with
``SeedSequence([2026, workload_id, layer, stream, b])``.  The same call always
yields the same bytes on any machine.
"""
from __future__ import annotations

import concurrent.futures as cf
import os

import numpy as np

__all__ = [
    "ROOT_SEED", "STREAM_Q", "STREAM_K", "STREAM_V", "STREAM_OUTLIER", "STREAM_PERM",
    "STREAM_LOGITS", "STREAM_PREFIX", "STREAM_TARGET", "CHUNK",
    "stream", "round_f32_to_bf16_bits", "bf16_bits_to_f32", "normal_bits",
    "normal_f32", "scatter_chunked", "paged_store", "ring_store", "ring_positions",
    "planted_logits", "planted_proposals", "NAN_BF16", "blocked_rows", "ROW_BLOCK",
]

ROOT_SEED = 2026
STREAM_Q, STREAM_K, STREAM_V, STREAM_OUTLIER, STREAM_PERM = 0, 1, 2, 3, 4
STREAM_LOGITS, STREAM_PREFIX, STREAM_TARGET = 5, 6, 7

#: tokens per KV chunk, the granularity the lucebox post pages its KV pool in
#: ("Three optimizations", item 1: cold 64-token chunks).
CHUNK = 64

#: bf16 quiet NaN, written into store slots that hold no position so that a
#: kernel that reads them without masking shows it.
NAN_BF16 = np.uint16(0x7FC0)


def stream(workload_id: int, layer: int, stream_id: int) -> np.random.Generator:
    return np.random.default_rng(
        np.random.SeedSequence([ROOT_SEED, int(workload_id), int(layer), int(stream_id)]))


def round_f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); returns the uint16 bit patterns.

    Finite inputs only (the generators never draw anything else).
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_f32(g: np.random.Generator, shape) -> np.ndarray:
    return g.standard_normal(size=shape, dtype=np.float32)


def normal_bits(g: np.random.Generator, shape) -> np.ndarray:
    """N(0,1) draws rounded to bf16; uint16 bit patterns."""
    return round_f32_to_bf16_bits(normal_f32(g, shape))


#: rows per independently seeded block of a large K/V draw
ROW_BLOCK = 8192


def _pool_size() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def blocked_rows(workload_id: int, layer: int, stream_id: int, n: int, row_shape, fn):
    """``[n, *row_shape]`` built block by block: block b (rows b*ROW_BLOCK ..) is
    ``fn(generator, rows)`` with its own generator seeded by
    ``SeedSequence([2026, workload_id, layer, stream_id, b])``.  Blocks are filled in a
    thread pool; the result does not depend on the number of threads."""
    nb = -(-n // ROW_BLOCK)
    first = None
    out = None

    def one(b):
        rows = min(ROW_BLOCK, n - b * ROW_BLOCK)
        g = np.random.default_rng(np.random.SeedSequence(
            [ROOT_SEED, int(workload_id), int(layer), int(stream_id), int(b)]))
        return b, fn(g, (rows, *row_shape))

    if nb == 0:
        return None
    with cf.ThreadPoolExecutor(_pool_size()) as ex:
        for b, arr in ex.map(one, range(nb)):
            if out is None:
                first = arr
                out = np.empty((n, *row_shape), dtype=first.dtype)
            out[b * ROW_BLOCK:b * ROW_BLOCK + len(arr)] = arr
    return out


def scatter_chunked(k_rows, v_rows, first_pos: int, slot_of_chunk, n_slots: int,
                    chunk: int = CHUNK, fill=None):
    """Scatter contiguous rows into the chunked store layout.

    ``k_rows``/``v_rows`` are ``[n][Hkv][D]`` for positions ``first_pos .. first_pos+n-1``.
    Returns ``K [n_slots][Hkv][chunk][D]`` and ``V [n_slots][Hkv][D][chunk]`` (V is stored
    dimension-major inside a chunk).  Position ``p`` goes to slot ``slot_of_chunk(p // chunk)``
    at offset ``p % chunk``.  Entries no row lands on are set to ``fill`` (default: NaN for
    bf16 bit patterns, NaN for float32).
    """
    k_rows = np.asarray(k_rows)
    v_rows = np.asarray(v_rows)
    n, hkv, d = k_rows.shape
    dt = k_rows.dtype
    if fill is None:
        fill = NAN_BF16 if dt == np.uint16 else np.float32(np.nan)
    K = np.empty((n_slots, hkv, chunk, d), dtype=dt)
    V = np.empty((n_slots, hkv, d, chunk), dtype=dt)
    if n == 0:
        K[...] = fill
        V[...] = fill
        return K, V
    c_first = first_pos // chunk
    c_last = (first_pos + n - 1) // chunk
    slots = np.array([slot_of_chunk(c) for c in range(c_first, c_last + 1)], dtype=np.int64)
    if len(np.unique(slots)) != len(slots):
        raise ValueError("two chunks of the span map to the same slot")
    covered = np.zeros(n_slots, dtype=bool)
    covered[slots] = True
    K[~covered] = fill
    V[~covered] = fill
    for idx, c in enumerate(range(c_first, c_last + 1)):
        lo = max(first_pos, c * chunk)
        hi = min(first_pos + n, (c + 1) * chunk)
        rk = k_rows[lo - first_pos:hi - first_pos]
        rv = v_rows[lo - first_pos:hi - first_pos]
        sl = slots[idx]
        if hi - lo == chunk:
            K[sl] = rk.transpose(1, 0, 2)          # [Hkv][chunk][D]
            V[sl] = rv.transpose(1, 2, 0)          # [Hkv][D][chunk]
        else:
            # a partially covered chunk keeps the fill value in its uncovered part
            K[sl] = fill
            V[sl] = fill
            K[sl, :, lo - c * chunk:hi - c * chunk, :] = rk.transpose(1, 0, 2)
            V[sl, :, :, lo - c * chunk:hi - c * chunk] = rv.transpose(1, 2, 0)
    return K, V


def paged_store(k_rows, v_rows, page_table, n_slots: int, chunk: int = CHUNK, fill=None):
    """Pool layout for positions ``0 .. n-1``: logical chunk ``c`` lives in slot ``page_table[c]``."""
    pt = np.asarray(page_table)
    return scatter_chunked(k_rows, v_rows, 0, lambda c: int(pt[c]), n_slots, chunk, fill)


def ring_positions(pos0: int, q_len: int, ring_size: int):
    """Positions the ring holds once the verify block is written: the last ``ring_size``
    positions up to ``pos0 + q_len - 1`` (none below 0)."""
    last = pos0 + q_len - 1
    first = max(0, last - ring_size + 1)
    return first, last


def ring_store(k_rows, v_rows, first_pos: int, ring_size: int, chunk: int = CHUNK, fill=None):
    """Ring layout: position ``p`` lives at slot ``p mod ring_size`` (chunk slot
    ``(p mod ring_size) // chunk``, offset ``p mod chunk``)."""
    if ring_size % chunk:
        raise ValueError("ring_size must be a multiple of the chunk size")
    n_ring_chunks = ring_size // chunk
    n = len(k_rows)
    if n > ring_size:
        raise ValueError("more rows than ring slots")
    # a span of ring_size positions that is not chunk-aligned touches one chunk slot twice
    # (head and tail of the same slot); place it in two passes.
    K = V = None
    c_first = first_pos // chunk
    c_last = (first_pos + n - 1) // chunk if n else c_first
    if n and c_last - c_first + 1 > n_ring_chunks:
        split = (c_first + 1) * chunk - first_pos
        K, V = scatter_chunked(k_rows[split:], v_rows[split:], first_pos + split,
                               lambda c: c % n_ring_chunks, n_ring_chunks, chunk, fill)
        slot = c_first % n_ring_chunks
        off = first_pos % chunk
        K[slot, :, off:off + split, :] = np.asarray(k_rows[:split]).transpose(1, 0, 2)
        V[slot, :, :, off:off + split] = np.asarray(v_rows[:split]).transpose(1, 2, 0)
        return K, V
    return scatter_chunked(k_rows, v_rows, first_pos, lambda c: c % n_ring_chunks,
                           n_ring_chunks, chunk, fill)


def planted_logits(g: np.random.Generator, n_rows: int, vocab: int, margin: float):
    """Logit rows ~ N(0,1) float32 whose argmax is a drawn index, unique by at least
    ``margin`` (``margin == 0``: by one float32 ulp).  Returns (logits, targets)."""
    L = normal_f32(g, (n_rows, vocab))
    t = g.integers(0, vocab, size=n_rows).astype(np.int64)
    if vocab == 1:
        return L, t.astype(np.int32)
    m32 = np.float32(margin)
    for r in range(n_rows):
        row = L[r]
        row[t[r]] = -np.inf
        second = row.max()
        top = np.float32(second + m32) if margin > 0 else np.nextafter(second, np.float32(np.inf))
        while margin > 0 and np.float32(top - second) < m32:
            top = np.nextafter(top, np.float32(np.inf))
        row[t[r]] = top
    return L, t.astype(np.int32)


def planted_proposals(g: np.random.Generator, targets, n_draft: int, vocab: int, accept: int):
    """Draft tokens that agree with ``targets`` on exactly the first ``accept`` positions."""
    t = np.asarray(targets, dtype=np.int64)
    prop = g.integers(0, vocab, size=n_draft).astype(np.int64)
    prop[:accept] = t[:accept]
    if accept < n_draft:
        if vocab < 2:
            raise ValueError("a mismatch needs a vocabulary of at least 2")
        prop[accept] = (t[accept] + 1 + g.integers(0, vocab - 1)) % vocab
    return prop.astype(np.int32)
