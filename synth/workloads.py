"""The verify-step workloads, built from the primitives in ``inputs``.

Named workloads (sizes in the names):

* ``contig_1k_f32``   - 16-token causal block after 1,008 prior tokens (context 1,024),
  8 query / 2 KV heads, head_dim 64, float32 Q/K/V ~ N(0,1); accept over [17 x 4096]
  logits with a drawn agreement prefix of 0..16.
* ``ring_w512_r2048`` - 16-token block at absolute position 30,000 over a wrapped
  2,048-slot ring, window 512, 16 / 4 heads, head_dim 128, bf16.
* ``paged_8k``        - 16-token block at context 8,192 over 128 permuted 64-token chunks.
* ``paged_256k``      - context 262,144, 4,096 permuted chunks, ~1% of K rows shifted by +4.
* ``stack_40l_131k``  - 40 layers: ``l % 4 != 3`` ring layers (block at 131,056), else paged
  layers at context 131,072 (2,048 permuted chunks); accept over [17 x 65536] logits with an
  argmax margin of at least 1e-3 and an agreement prefix ~ Binomial(16, 9/16).

Batched prefill (1,024-token blocks through the same stores, 16 / 4 heads, head_dim 128, bf16):

* ``prefill_pool_8k``   - block after 8,192 prior tokens (context 9,216), 144 permuted chunks.
* ``prefill_ring_w512`` - block at absolute position 30,000 over the wrapped 2,048-slot ring,
  window 512.
* ``prefill_pool_131k`` - block ending at context 131,072 (2,048 permuted chunks): the paged
  layers of the 40-layer stack, one prefill block further on.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

from .inputs import (CHUNK, STREAM_K, blocked_rows, STREAM_LOGITS, STREAM_OUTLIER, STREAM_PERM,
                     STREAM_PREFIX, STREAM_Q, STREAM_V, normal_bits, normal_f32,
                     paged_store, planted_logits, planted_proposals,
                     round_f32_to_bf16_bits, ring_positions, ring_store, stream)

__all__ = [
    "AttnCase", "AcceptCase", "WORKLOAD_IDS", "contig_case", "ring_case", "paged_case",
    "accept_case", "workload", "stack_layer_kind", "STACK_LAYERS",
]

#: seed ids of the named workloads
WORKLOAD_IDS = {
    "contig_1k_f32": 1, "ring_w512_r2048": 2, "paged_8k": 3, "paged_256k": 4,
    "stack_40l_131k": 5, "prefill_pool_8k": 6, "prefill_ring_w512": 7, "prefill_pool_131k": 8,
}
STACK_LAYERS = 40


@dataclass
class AttnCase:
    kind: str                     # "contig" | "ring" | "paged"
    dtype: str                    # "bf16" (uint16 bit patterns) | "f32"
    q: np.ndarray                 # [q_len][Hq][D]
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    q_len: int
    scale: float
    window: int = 0               # 0: full causal
    ctx_len: int = 0              # positions 0 .. ctx_len-1 exist (query i at ctx_len-q_len+i)
    rows_first: int = 0           # position of k_rows[0]
    k_rows: Optional[np.ndarray] = None   # contiguous [n][Hkv][D] (kept unless dropped)
    v_rows: Optional[np.ndarray] = None
    # ring store
    pos0: int = 0
    ring_size: int = 0
    ring_head: int = 0
    k_ring: Optional[np.ndarray] = None   # [ring_size/64][Hkv][64][D]
    v_ring: Optional[np.ndarray] = None   # [ring_size/64][Hkv][D][64]
    # paged store
    page_table: Optional[np.ndarray] = None
    n_slots: int = 0
    chunk: int = CHUNK
    k_pool: Optional[np.ndarray] = None   # [n_slots][Hkv][64][D]
    v_pool: Optional[np.ndarray] = None   # [n_slots][Hkv][D][64]
    meta: dict = field(default_factory=dict)

    @property
    def kv_bytes(self) -> int:
        """Bytes of K and V the method must read once: every attended position, per KV head."""
        n = self.attended_positions()
        esz = 2 if self.dtype == "bf16" else 4
        return 2 * n * self.n_kv_heads * self.head_dim * esz

    def attended_positions(self) -> int:
        first_q = self.ctx_len - self.q_len
        lo = max(0, first_q - self.window + 1) if self.window else 0
        return self.ctx_len - lo


@dataclass
class AcceptCase:
    logits: np.ndarray            # [n_draft+1][vocab] float32
    proposals: np.ndarray         # [n_draft] int32
    planted_accept: int
    planted_targets: np.ndarray   # [n_draft+1] int32, the argmax of each row by construction
    n_draft: int
    vocab: int


def _draw(wid, layer, sid, shape, dtype):
    g = stream(wid, layer, sid)
    return normal_bits(g, shape) if dtype == "bf16" else normal_f32(g, shape)


def _kv_rows(wid, layer, n, hkv, d, dtype, outlier_rate=0.0, outlier_shift=4.0):
    """K and V rows [n][Hkv][D] ~ N(0,1); with ``outlier_rate`` > 0 each (row, KV head) of K
    is shifted by +outlier_shift on every element with that probability (before rounding)."""
    if dtype == "f32":
        return (blocked_rows(wid, layer, STREAM_K, n, (hkv, d), normal_f32),
                blocked_rows(wid, layer, STREAM_V, n, (hkv, d), normal_f32))

    def k_block(g, shape):
        x = normal_f32(g, shape)
        if outlier_rate > 0:
            sel = g.random(shape[:2]) < outlier_rate
            x[sel] += np.float32(outlier_shift)
        return round_f32_to_bf16_bits(x)

    k = blocked_rows(wid, layer, STREAM_K, n, (hkv, d), k_block)
    v = blocked_rows(wid, layer, STREAM_V, n, (hkv, d), normal_bits)
    return k, v


def _perm(wid, layer, n_slots, n_chunks, how):
    if how == "identity":
        return np.arange(n_chunks, dtype=np.int32)
    if how == "reversed":
        return (n_slots - 1 - np.arange(n_chunks)).astype(np.int32)
    if how == "seeded":
        return stream(wid, layer, STREAM_PERM).permutation(n_slots)[:n_chunks].astype(np.int32)
    raise ValueError(how)


def contig_case(wid, layer, ctx_len, q_len, hq, hkv, d, dtype, window=0):
    q = _draw(wid, layer, STREAM_Q, (q_len, hq, d), dtype)
    k, v = _kv_rows(wid, layer, ctx_len, hkv, d, dtype)
    return AttnCase("contig", dtype, q, hq, hkv, d, q_len, 1.0 / np.sqrt(d), window, ctx_len,
                    0, k, v)


def ring_case(wid, layer, pos0, q_len, hq, hkv, d, ring_size=2048, window=512, dtype="bf16",
              keep_rows=True):
    q = _draw(wid, layer, STREAM_Q, (q_len, hq, d), dtype)
    first, last = ring_positions(pos0, q_len, ring_size)
    k, v = _kv_rows(wid, layer, last - first + 1, hkv, d, dtype)
    kr, vr = ring_store(k, v, first, ring_size)
    c = AttnCase("ring", dtype, q, hq, hkv, d, q_len, 1.0 / np.sqrt(d), window, pos0 + q_len,
                 first, k if keep_rows else None, v if keep_rows else None,
                 pos0=pos0, ring_size=ring_size, ring_head=pos0 % ring_size, k_ring=kr, v_ring=vr)
    return c


def paged_case(wid, layer, ctx_len, q_len, hq, hkv, d, n_slots=None, perm="seeded",
               outlier_rate=0.0, dtype="bf16", keep_rows=True, chunk=CHUNK):
    n_chunks = -(-ctx_len // chunk)
    n_slots = n_chunks if n_slots is None else n_slots
    q = _draw(wid, layer, STREAM_Q, (q_len, hq, d), dtype)
    k, v = _kv_rows(wid, layer, ctx_len, hkv, d, dtype, outlier_rate)
    pt = _perm(wid, layer, n_slots, n_chunks, perm)
    kp, vp = paged_store(k, v, pt, n_slots, chunk)
    return AttnCase("paged", dtype, q, hq, hkv, d, q_len, 1.0 / np.sqrt(d), 0, ctx_len, 0,
                    k if keep_rows else None, v if keep_rows else None,
                    page_table=pt, n_slots=n_slots, chunk=chunk, k_pool=kp, v_pool=vp)


def accept_case(wid, layer, n_draft, vocab, margin, prefix="uniform", accept=None):
    g = stream(wid, layer, STREAM_LOGITS)
    L, t = planted_logits(g, n_draft + 1, vocab, margin)
    gp = stream(wid, layer, STREAM_PREFIX)
    if accept is None:
        if prefix == "uniform":
            accept = int(gp.integers(0, n_draft + 1))
        elif prefix == "binomial":
            accept = int(gp.binomial(n_draft, 9.0 / 16.0))
        else:
            raise ValueError(prefix)
    if vocab < 2:
        accept = n_draft
    prop = planted_proposals(gp, t, n_draft, vocab, accept)
    return AcceptCase(L, prop, accept, t, n_draft, vocab)


def stack_layer_kind(layer: int) -> str:
    """Three in four layers are sliding-window ring layers; every fourth is a paged
    full-attention layer."""
    return "paged" if layer % 4 == 3 else "ring"


def workload(name: str, layer: int = 0, keep_rows: bool = True):
    """The named workload's inputs: ``(attention case(s), accept case or None)``.

    For ``stack_40l_131k`` pass ``layer`` to get one layer's attention case; the accept
    case is the same for every layer.
    """
    wid = WORKLOAD_IDS[name]
    if name == "contig_1k_f32":
        return (contig_case(wid, 0, 1024, 16, 8, 2, 64, "f32"),
                accept_case(wid, 0, 16, 4096, 0.0, "uniform"))
    if name == "ring_w512_r2048":
        return ring_case(wid, 0, 30000, 16, 16, 4, 128, 2048, 512, keep_rows=keep_rows), None
    if name == "paged_8k":
        return paged_case(wid, 0, 8192, 16, 16, 4, 128, keep_rows=keep_rows), None
    if name == "paged_256k":
        return paged_case(wid, 0, 262144, 16, 16, 4, 128, n_slots=4096, outlier_rate=0.01,
                          keep_rows=keep_rows), None
    if name == "stack_40l_131k":
        if stack_layer_kind(layer) == "ring":
            a = ring_case(wid, layer, 131072 - 16, 16, 16, 4, 128, 2048, 512, keep_rows=keep_rows)
        else:
            a = paged_case(wid, layer, 131072, 16, 16, 4, 128, n_slots=2048, keep_rows=keep_rows)
        return a, accept_case(wid, 0, 16, 65536, 1e-3, "binomial")
    if name == "prefill_pool_8k":
        return paged_case(wid, 0, 9216, 1024, 16, 4, 128, keep_rows=keep_rows), None
    if name == "prefill_ring_w512":
        return ring_case(wid, 0, 30000, 1024, 16, 4, 128, 2048, 512, keep_rows=keep_rows), None
    if name == "prefill_pool_131k":
        return paged_case(wid, 0, 131072, 1024, 16, 4, 128, n_slots=2048,
                          keep_rows=keep_rows), None
    raise KeyError(name)
