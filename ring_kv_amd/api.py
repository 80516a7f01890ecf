"""Torch-tensor front end of libring_kv.  Argument marshalling only: every step of the verify
path runs in the library's HIP kernels; torch supplies device memory and the stream.

Layouts are those of include/ring_kv.h: Q [q_len][Hq][D]; chunked K [slots][Hkv][64][D] and
V [slots][Hkv][D][64] (bf16); out [q_len][Hq][D] and lse [q_len][Hq] float32.
"""
from __future__ import annotations

import ctypes
from typing import Optional, Tuple

import torch

from ._lib import RKV_BF16, RKV_F32, AttnDims, check, lib

CHUNK = 64
RKV_MAX_APPEND_CHUNKS = 17


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _form(t, name: str, dtype=None, shape=None):
    """Type, dtype, contiguity and shape of one tensor argument; None in `shape` matches any
    size.  The library takes plain pointers and trusts the sizes it is given, so every buffer
    it reads or writes is checked here against the sizes the call will use."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if shape is not None and (t.dim() != len(shape) or
                              any(e is not None and n != e for n, e in zip(t.shape, shape))):
        want = "[" + "][".join("*" if e is None else str(e) for e in shape) + "]"
        raise ValueError(f"{name} has shape {list(t.shape)}, expected {want}")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise ValueError(f"{name} has dtype {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _on(device, **tensors):
    """Every given tensor (None skipped) is a device tensor on `device`."""
    for name, t in tensors.items():
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if t.device != device:
            raise ValueError(f"{name} is on {t.device}, expected {device}")


def _stream(stream, device):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _dims(q: torch.Tensor, n_kv_heads: int, scale: float) -> AttnDims:
    q_len, hq, d = q.shape
    dt = RKV_BF16 if q.dtype == torch.bfloat16 else RKV_F32
    return AttnDims(q_len, hq, n_kv_heads, d, float(scale), dt)


def _workspace(nbytes: int, device, ws: Optional[torch.Tensor]):
    """The caller's workspace (checked to hold nbytes), or a new one of nbytes."""
    if nbytes == 0:
        return None, 0
    if ws is not None:
        _form(ws, "workspace")
        _on(device, workspace=ws)
        if ws.numel() * ws.element_size() < nbytes:
            raise ValueError(f"workspace holds {ws.numel() * ws.element_size()} bytes, need {nbytes}")
        return ws, ws.numel() * ws.element_size()
    return torch.empty(nbytes, dtype=torch.uint8, device=device), nbytes


# Counter bytes at the start of a full-size ring workspace (RKV_RING_COUNTER_BYTES).
RING_COUNTER_BYTES = 8192


def _ring_workspace(full: int, device, ws: Optional[torch.Tensor]):
    """A ring call's workspace.  full = verify_attn_ring_workspace_bytes(): with it (counters
    zeroed before first use, which the caller owns) the layer runs as one launch; a workspace of
    only the partials (full - RING_COUNTER_BYTES) merges in a second launch.  Without a caller
    workspace a fresh one of the partials' size is used (nothing to zero inside the call)."""
    if full == 0:
        return None, 0
    return _workspace(full - RING_COUNTER_BYTES, device, ws)


def _outputs(q_len: int, hq: int, d: int, device, out, lse, want_lse):
    if out is None:
        out = torch.empty((q_len, hq, d), dtype=torch.float32, device=device)
    if lse is None and want_lse:
        lse = torch.empty((q_len, hq), dtype=torch.float32, device=device)
    _form(out, "out", torch.float32, (q_len, hq, d))
    if lse is not None:
        _form(lse, "lse", torch.float32, (q_len, hq))
    _on(device, out=out, lse=lse)
    return out, lse


def _chunked(k, v, kname: str, vname: str, d: Optional[int] = None, n_kv: Optional[int] = None):
    """A chunked K/V store: K [slots][Hkv][64][D] and V [slots][Hkv][D][64] bf16 of matching
    sizes.  Returns (slots, Hkv, D)."""
    _form(k, kname, torch.bfloat16, (None, n_kv, CHUNK, d))
    n, hkv, _, dk = k.shape
    _form(v, vname, torch.bfloat16, (n, hkv, dk, CHUNK))
    return n, hkv, dk


def _rows_pair(k, v, kname: str, vname: str):
    """Rows K, V [n][Hkv][D] bf16 of the same shape.  Returns (n, Hkv, D)."""
    _form(k, kname, torch.bfloat16, (None, None, None))
    _form(v, vname, torch.bfloat16, tuple(k.shape))
    return tuple(k.shape)


def verify_attn_paged(q, k_pool, v_pool, page_table, ctx_len: int, *, num_splits: int = 0,
                      scale: float = 0.0, out=None, lse=None, want_lse: bool = True,
                      workspace=None, stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Full-attention verify block over the paged pool of 64-token chunks."""
    _form(q, "q", torch.bfloat16, (None, None, None))
    q_len, hq, d = q.shape
    n_slots, hkv, _ = _chunked(k_pool, v_pool, "k_pool", "v_pool", d)
    _form(page_table, "page_table", torch.int32, (None,))
    dev = q.device
    out, lse = _outputs(q_len, hq, d, dev, out, lse, want_lse)
    _on(dev, q=q, k_pool=k_pool, v_pool=v_pool, page_table=page_table)
    dims = _dims(q, hkv, scale)
    L = lib()
    ws, wsb = _workspace(L.verify_attn_paged_workspace_bytes(ctypes.byref(dims), ctx_len, CHUNK,
                                                             num_splits), dev, workspace)
    check("verify_attn_paged", L.verify_attn_paged(
        ctypes.byref(dims), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(page_table),
        page_table.numel(), n_slots, CHUNK, ctx_len, num_splits, _ptr(ws), wsb, _ptr(out),
        _ptr(lse), _stream(stream, dev)))
    return out, lse


def verify_attn_paged_auto_splits(n_q_heads: int, n_kv_heads: int, head_dim: int, q_len: int,
                                  ctx_len: int) -> int:
    dims = AttnDims(q_len, n_q_heads, n_kv_heads, head_dim, 0.0, RKV_BF16)
    return lib().verify_attn_paged_auto_splits(ctypes.byref(dims), ctx_len, CHUNK)


def verify_attn_paged_partial(q, k_pool, v_pool, page_table, ctx_len: int, num_splits: int, *,
                              scale: float = 0.0, part_out=None, part_lse=None, stream=None):
    """Phase one of the paged call: per split of the chunk range, the normalised output
    [Hkv][S][rows][D] and the split's lse [Hkv][S][rows]."""
    _form(q, "q", torch.bfloat16, (None, None, None))
    q_len, hq, d = q.shape
    n_slots, hkv, _ = _chunked(k_pool, v_pool, "k_pool", "v_pool", d)
    _form(page_table, "page_table", torch.int32, (None,))
    if num_splits < 1 or hq % hkv != 0:
        raise ValueError("num_splits must be >= 1 and n_q_heads a multiple of n_kv_heads")
    rows = q_len * (hq // hkv)
    dev = q.device
    if part_out is None:
        part_out = torch.empty((hkv, num_splits, rows, d), dtype=torch.float32, device=dev)
    if part_lse is None:
        part_lse = torch.empty((hkv, num_splits, rows), dtype=torch.float32, device=dev)
    _form(part_out, "part_out", torch.float32, (hkv, num_splits, rows, d))
    _form(part_lse, "part_lse", torch.float32, (hkv, num_splits, rows))
    _on(dev, q=q, k_pool=k_pool, v_pool=v_pool, page_table=page_table, part_out=part_out,
        part_lse=part_lse)
    dims = _dims(q, hkv, scale)
    check("verify_attn_paged_partial", lib().verify_attn_paged_partial(
        ctypes.byref(dims), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(page_table),
        page_table.numel(), n_slots, CHUNK, ctx_len, num_splits, _ptr(part_out), _ptr(part_lse),
        _stream(stream, dev)))
    return part_out, part_lse


def attn_merge_partials(part_out, part_lse, q_len: int, n_q_heads: int, *, out=None, lse=None,
                        want_lse: bool = True, stream=None):
    """Log-sum-exp merge of split partials (layout of verify_attn_paged_partial)."""
    _form(part_out, "part_out", torch.float32, (None, None, None, None))
    hkv, S, rows, d = part_out.shape
    _form(part_lse, "part_lse", torch.float32, (hkv, S, rows))
    if n_q_heads % hkv != 0 or rows != q_len * (n_q_heads // hkv):
        raise ValueError(f"partials of {rows} rows per KV head do not match q_len {q_len} x "
                         f"{n_q_heads} query heads over {hkv} KV heads")
    dev = part_out.device
    out, lse = _outputs(q_len, n_q_heads, d, dev, out, lse, want_lse)
    _on(dev, part_out=part_out, part_lse=part_lse)
    dims = AttnDims(q_len, n_q_heads, hkv, d, 0.0, RKV_BF16)
    check("attn_merge_partials", lib().attn_merge_partials(
        ctypes.byref(dims), S, _ptr(part_out), _ptr(part_lse), _ptr(out), _ptr(lse),
        _stream(stream, dev)))
    return out, lse


def verify_attn_ring(q, k_ring, v_ring, pos0: int, window: int, *, num_splits: int = 0,
                     scale: float = 0.0, out=None, lse=None, want_lse: bool = True,
                     workspace=None, stream=None):
    """Sliding-window verify block over the position ring (slot = pos mod ring_size).
    workspace: a persistent uint8 device buffer of verify_attn_ring_workspace_bytes() bytes,
    zeroed once before its first use, runs the layer as one launch; without one, a fresh buffer
    of the partials alone is used and a second launch merges them (the same bits)."""
    _form(q, "q", torch.bfloat16, (None, None, None))
    q_len, hq, d = q.shape
    n_chunks, hkv, _ = _chunked(k_ring, v_ring, "k_ring", "v_ring", d)
    dev = q.device
    out, lse = _outputs(q_len, hq, d, dev, out, lse, want_lse)
    _on(dev, q=q, k_ring=k_ring, v_ring=v_ring)
    ring_size = n_chunks * CHUNK
    dims = _dims(q, hkv, scale)
    L = lib()
    ws, wsb = _ring_workspace(L.verify_attn_ring_workspace_bytes(ctypes.byref(dims), ring_size,
                                                                 window, num_splits), dev, workspace)
    check("verify_attn_ring", L.verify_attn_ring(
        ctypes.byref(dims), _ptr(q), _ptr(k_ring), _ptr(v_ring), pos0, pos0 % ring_size,
        ring_size, window, num_splits, _ptr(ws), wsb, _ptr(out), _ptr(lse), _stream(stream, dev)))
    return out, lse


def decode_attn_ref_layout(q, k, v, ctx_len: int, window: int = 0, *, num_splits: int = 0,
                           scale: float = 0.0, out=None, lse=None, want_lse: bool = True,
                           workspace=None, stream=None):
    """Verify/decode attention over the contiguous layout K, V [ctx][Hkv][D] (f32 or bf16)."""
    _form(q, "q", (torch.float32, torch.bfloat16), (None, None, None))
    q_len, hq, d = q.shape
    _form(k, "k", q.dtype, (None, None, d))
    _form(v, "v", q.dtype, tuple(k.shape))
    hkv = k.shape[1]
    if k.shape[0] < ctx_len:
        raise ValueError("k, v hold fewer than ctx_len rows")
    dev = q.device
    out, lse = _outputs(q_len, hq, d, dev, out, lse, want_lse)
    _on(dev, q=q, k=k, v=v)
    dims = _dims(q, hkv, scale)
    L = lib()
    ws, wsb = _workspace(L.decode_attn_ref_layout_workspace_bytes(ctypes.byref(dims), ctx_len,
                                                                  num_splits), dev, workspace)
    check("decode_attn_ref_layout", L.decode_attn_ref_layout(
        ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), ctx_len, window, num_splits, _ptr(ws), wsb,
        _ptr(out), _ptr(lse), _stream(stream, dev)))
    return out, lse


def verify_accept(logits, proposals, *, accept_len=None, committed=None, row_argmax=None,
                  want_argmax: bool = True, workspace=None, stream=None):
    """Greedy acceptance: (accept_len [1], committed [k+1] (-1 after a+1), row_argmax [k+1])."""
    _form(proposals, "proposals", torch.int32, (None,))
    k = proposals.numel()
    _form(logits, "logits", torch.float32, (k + 1, None))
    vocab = logits.shape[1]
    dev = logits.device
    if accept_len is None:
        accept_len = torch.empty(1, dtype=torch.int32, device=dev)
    if committed is None:
        committed = torch.empty(k + 1, dtype=torch.int32, device=dev)
    if row_argmax is None and want_argmax:
        row_argmax = torch.empty(k + 1, dtype=torch.int32, device=dev)
    _form(accept_len, "accept_len", torch.int32, (1,))
    _form(committed, "committed", torch.int32, (k + 1,))
    if row_argmax is not None:
        _form(row_argmax, "row_argmax", torch.int32, (k + 1,))
    _on(dev, logits=logits, proposals=proposals, accept_len=accept_len, committed=committed,
        row_argmax=row_argmax)
    L = lib()
    ws, wsb = _workspace(L.verify_accept_workspace_bytes(k, vocab), dev, workspace)
    check("verify_accept", L.verify_accept(
        _ptr(logits), k, vocab, _ptr(proposals), _ptr(accept_len), _ptr(committed),
        _ptr(row_argmax), _ptr(ws), wsb, _stream(stream, dev)))
    return accept_len, committed, row_argmax


def ref_layout_to_ring(k_src, v_src, pos_first: int, k_ring, v_ring, *, stream=None):
    """Write rows k_src, v_src [n][Hkv][D] (positions pos_first..) into the ring."""
    n, hkv, d = _rows_pair(k_src, v_src, "k_src", "v_src")
    n_chunks, _, _ = _chunked(k_ring, v_ring, "k_ring", "v_ring", d, hkv)
    dev = k_src.device
    _on(dev, k_src=k_src, v_src=v_src, k_ring=k_ring, v_ring=v_ring)
    check("ref_layout_to_ring", lib().ref_layout_to_ring(
        _ptr(k_src), _ptr(v_src), pos_first, n, hkv, d, RKV_BF16, _ptr(k_ring), _ptr(v_ring),
        n_chunks * CHUNK, _stream(stream, dev)))


def ref_layout_to_paged(k_src, v_src, pos_first: int, k_pool, v_pool, page_table, *,
                        stream=None):
    """Write rows k_src, v_src [n][Hkv][D] (positions pos_first..) into the paged pool."""
    n, hkv, d = _rows_pair(k_src, v_src, "k_src", "v_src")
    n_slots, _, _ = _chunked(k_pool, v_pool, "k_pool", "v_pool", d, hkv)
    _form(page_table, "page_table", torch.int32, (None,))
    dev = k_src.device
    _on(dev, k_src=k_src, v_src=v_src, k_pool=k_pool, v_pool=v_pool, page_table=page_table)
    check("ref_layout_to_paged", lib().ref_layout_to_paged(
        _ptr(k_src), _ptr(v_src), pos_first, n, hkv, d, RKV_BF16, _ptr(k_pool), _ptr(v_pool),
        _ptr(page_table), page_table.numel(), n_slots, CHUNK, _stream(stream, dev)))


class Pager:
    """The library's host-side pager of a paged pool (rkv_pager_*): slot free list and a host
    copy of the page table for one sequence; reserve -> append -> commit per verify block."""

    def __init__(self, n_slots: int, n_table: int):
        self._L = lib()
        self._p = self._L.rkv_pager_create(n_slots, n_table)
        if not self._p:
            raise ValueError("rkv_pager_create: sizes must be >= 1")
        self.n_slots, self.n_table = n_slots, n_table

    def close(self):
        if self._p:
            self._L.rkv_pager_destroy(self._p)
            self._p = None

    def __del__(self):
        self.close()

    @property
    def ctx_len(self) -> int:
        return int(self._L.rkv_pager_ctx_len(self._p))

    @property
    def free_slots(self) -> int:
        return int(self._L.rkv_pager_free_slots(self._p))

    def table(self, n: Optional[int] = None):
        """Host copy of the first n table entries (-1: no slot) as a list."""
        n = self.n_table if n is None else n
        buf = (ctypes.c_int32 * max(1, n))()
        check("rkv_pager_table", self._L.rkv_pager_table(self._p, buf, n))
        return list(buf)[:n]

    def reserve(self, n: int):
        """Slots for the chunks the next n positions start: (first_chunk, [slots])."""
        first, k = ctypes.c_int32(), ctypes.c_int32()
        slots = (ctypes.c_int32 * RKV_MAX_APPEND_CHUNKS)()
        check("rkv_pager_reserve", self._L.rkv_pager_reserve(
            self._p, n, ctypes.byref(first), ctypes.byref(k), slots))
        return first.value, list(slots)[:k.value]

    def commit(self, n_keep: int):
        check("rkv_pager_commit", self._L.rkv_pager_commit(self._p, n_keep))

    def evict(self, chunk_ids):
        """Page whole committed chunks out: their slots (to copy out with kv_page_out before
        any reuse), in the order given."""
        n = len(chunk_ids)
        ids = (ctypes.c_int32 * max(1, n))(*chunk_ids)
        slots = (ctypes.c_int32 * max(1, n))()
        check("rkv_pager_evict", self._L.rkv_pager_evict(self._p, ids, n, slots))
        return list(slots)[:n]

    def restore(self, chunk_ids):
        """Give paged-out chunks slots again (to copy in with kv_page_in), in the order given."""
        n = len(chunk_ids)
        ids = (ctypes.c_int32 * max(1, n))(*chunk_ids)
        slots = (ctypes.c_int32 * max(1, n))()
        check("rkv_pager_restore", self._L.rkv_pager_restore(self._p, ids, n, slots))
        return list(slots)[:n]

    def resident(self):
        """(chunk ids, slots) of the chunks that have a slot, in increasing chunk order."""
        k = self._L.rkv_pager_resident(self._p, None, None, 0)
        if k < 0:
            check("rkv_pager_resident", k)
        ids = (ctypes.c_int32 * max(1, k))()
        slots = (ctypes.c_int32 * max(1, k))()
        self._L.rkv_pager_resident(self._p, ids, slots, k)
        return list(ids)[:k], list(slots)[:k]


def verify_kv_append_ring(k_new, v_new, pos_first: int, k_ring, v_ring, *, stream=None):
    """Append a verify block's rows k_new, v_new [n][Hkv][D] (positions pos_first..) to the
    ring at slot pos mod ring_size."""
    n, hkv, d = _rows_pair(k_new, v_new, "k_new", "v_new")
    n_chunks, _, _ = _chunked(k_ring, v_ring, "k_ring", "v_ring", d, hkv)
    dev = k_new.device
    _on(dev, k_new=k_new, v_new=v_new, k_ring=k_ring, v_ring=v_ring)
    check("verify_kv_append_ring", lib().verify_kv_append_ring(
        _ptr(k_new), _ptr(v_new), n, pos_first, hkv, d, _ptr(k_ring), _ptr(v_ring),
        n_chunks * CHUNK, _stream(stream, dev)))


def verify_kv_append_paged(k_new, v_new, ctx_len: int, k_pool, v_pool, page_table,
                           first_chunk: int, new_slots, *, stream=None):
    """Append a verify block's rows (positions ctx_len..) to the pool; the chunks the block
    starts (from Pager.reserve) get new_slots, written into the device page table too."""
    n, hkv, d = _rows_pair(k_new, v_new, "k_new", "v_new")
    n_slots, _, _ = _chunked(k_pool, v_pool, "k_pool", "v_pool", d, hkv)
    _form(page_table, "page_table", torch.int32, (None,))
    dev = k_new.device
    _on(dev, k_new=k_new, v_new=v_new, k_pool=k_pool, v_pool=v_pool, page_table=page_table)
    slots = (ctypes.c_int32 * max(1, len(new_slots)))(*new_slots)
    check("verify_kv_append_paged", lib().verify_kv_append_paged(
        _ptr(k_new), _ptr(v_new), n, ctx_len, hkv, d, _ptr(k_pool), _ptr(v_pool),
        _ptr(page_table), page_table.numel(), n_slots, first_chunk, len(new_slots),
        slots, _stream(stream, dev)))


def _host_stores(k_host, v_host, hkv: int, d: int) -> int:
    """Host chunk stores laid out like the pool's slots: K [n_host][Hkv][64][D] and V
    [n_host][Hkv][D][64] bf16 host tensors (pinned for asynchronous copies).  Returns n_host."""
    for t, name in ((k_host, "k_host"), (v_host, "v_host")):
        if not isinstance(t, torch.Tensor) or t.is_cuda:
            raise ValueError(f"{name} must be a host tensor (pinned for asynchronous copies)")
    _chunked(k_host, v_host, "k_host", "v_host", d, hkv)
    return k_host.shape[0]


def kv_page_out(k_pool, v_pool, slots, chunk_ids, k_host, v_host, *, workspace=None,
                stream=None):
    """Copy pool slots[i] to host entries chunk_ids[i] (K and V, bit-exact), asynchronously on
    the stream; k_host [n_host][Hkv][64][D], v_host [n_host][Hkv][D][64] host tensors."""
    n_slots, hkv, d = _chunked(k_pool, v_pool, "k_pool", "v_pool")
    n_host = _host_stores(k_host, v_host, hkv, d)
    dev = k_pool.device
    _on(dev, k_pool=k_pool, v_pool=v_pool)
    n = len(slots)
    if len(chunk_ids) != n:
        raise ValueError("slots and chunk_ids differ in length")
    L = lib()
    ws, wsb = _workspace(L.kv_page_workspace_bytes(hkv, d, n), dev, workspace)
    sl = (ctypes.c_int32 * max(1, n))(*slots)
    ci = (ctypes.c_int32 * max(1, n))(*chunk_ids)
    check("kv_page_out", L.kv_page_out(
        _ptr(k_pool), _ptr(v_pool), hkv, d, n_slots, sl, ci, n,
        ctypes.c_void_p(k_host.data_ptr()), ctypes.c_void_p(v_host.data_ptr()),
        n_host, _ptr(ws), wsb, _stream(stream, dev)))
    return ws


def kv_page_in(k_host, v_host, chunk_ids, slots, k_pool, v_pool, *, workspace=None,
               stream=None):
    """Copy host entries chunk_ids[i] into pool slots[i] (K and V, bit-exact), asynchronously
    on the stream."""
    n_slots, hkv, d = _chunked(k_pool, v_pool, "k_pool", "v_pool")
    n_host = _host_stores(k_host, v_host, hkv, d)
    dev = k_pool.device
    _on(dev, k_pool=k_pool, v_pool=v_pool)
    n = len(slots)
    if len(chunk_ids) != n:
        raise ValueError("slots and chunk_ids differ in length")
    L = lib()
    ws, wsb = _workspace(L.kv_page_workspace_bytes(hkv, d, n), dev, workspace)
    sl = (ctypes.c_int32 * max(1, n))(*slots)
    ci = (ctypes.c_int32 * max(1, n))(*chunk_ids)
    check("kv_page_in", L.kv_page_in(
        ctypes.c_void_p(k_host.data_ptr()), ctypes.c_void_p(v_host.data_ptr()), n_host,
        ci, sl, n, _ptr(k_pool), _ptr(v_pool), hkv, d, n_slots, _ptr(ws), wsb,
        _stream(stream, dev)))
    return ws


def verify_attn_paged_resident(q, k_pool, v_pool, d_slots, chunk_ids, ctx_len: int, *,
                               num_splits: int = 0, scale: float = 0.0, out=None, lse=None,
                               want_lse: bool = True, workspace=None, stream=None):
    """Full-attention attention of the block over the resident chunks only: chunk_ids (host
    list, increasing) read from the device slot list d_slots."""
    _form(q, "q", torch.bfloat16, (None, None, None))
    q_len, hq, d = q.shape
    n_slots, hkv, _ = _chunked(k_pool, v_pool, "k_pool", "v_pool", d)
    n_res = len(chunk_ids)
    _form(d_slots, "d_slots", torch.int32, (n_res,))
    dev = q.device
    out, lse = _outputs(q_len, hq, d, dev, out, lse, want_lse)
    _on(dev, q=q, k_pool=k_pool, v_pool=v_pool, d_slots=d_slots)
    dims = _dims(q, hkv, scale)
    L = lib()
    # the call runs over n_res chunks: its splits and workspace are those of 64 * n_res positions
    ws, wsb = _workspace(L.verify_attn_paged_workspace_bytes(ctypes.byref(dims), CHUNK * n_res,
                                                             CHUNK, num_splits), dev, workspace)
    ci = (ctypes.c_int32 * max(1, n_res))(*chunk_ids)
    check("verify_attn_paged_resident", L.verify_attn_paged_resident(
        ctypes.byref(dims), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(d_slots), ci, n_res,
        n_slots, ctx_len, num_splits, _ptr(ws), wsb, _ptr(out), _ptr(lse), _stream(stream, dev)))
    return out, lse


def _pos_tensor(d_pos, device):
    """The device-resident block position: one int64 on the calls' device."""
    _form(d_pos, "d_pos", torch.int64, (1,))
    _on(device, d_pos=d_pos)


def verify_attn_ring_dev(q, k_ring, v_ring, d_pos, pos_cap: int, window: int, *,
                         num_splits: int = 0, scale: float = 0.0, out=None, lse=None,
                         want_lse: bool = True, workspace=None, stream=None):
    """verify_attn_ring with the block's first position read from d_pos (int64 [1], device)
    when the stream runs the call: a captured graph replays at whatever *d_pos holds."""
    _form(q, "q", torch.bfloat16, (None, None, None))
    q_len, hq, d = q.shape
    n_chunks, hkv, _ = _chunked(k_ring, v_ring, "k_ring", "v_ring", d)
    dev = q.device
    _pos_tensor(d_pos, dev)
    out, lse = _outputs(q_len, hq, d, dev, out, lse, want_lse)
    _on(dev, q=q, k_ring=k_ring, v_ring=v_ring)
    ring_size = n_chunks * CHUNK
    dims = _dims(q, hkv, scale)
    L = lib()
    ws, wsb = _ring_workspace(L.verify_attn_ring_workspace_bytes(ctypes.byref(dims), ring_size,
                                                                 window, num_splits), dev, workspace)
    check("verify_attn_ring_dev", L.verify_attn_ring_dev(
        ctypes.byref(dims), _ptr(q), _ptr(k_ring), _ptr(v_ring), _ptr(d_pos), pos_cap, ring_size,
        window, num_splits, _ptr(ws), wsb, _ptr(out), _ptr(lse), _stream(stream, dev)))
    return out, lse


def verify_attn_paged_dev(q, k_pool, v_pool, page_table, d_pos, pos_cap: int, *,
                          num_splits: int = 0, scale: float = 0.0, out=None, lse=None,
                          want_lse: bool = True, workspace=None, stream=None):
    """verify_attn_paged at context *d_pos + q_len, read from the device when the stream runs
    the call; splits and workspace cover every position up to pos_cap."""
    _form(q, "q", torch.bfloat16, (None, None, None))
    q_len, hq, d = q.shape
    n_slots, hkv, _ = _chunked(k_pool, v_pool, "k_pool", "v_pool", d)
    _form(page_table, "page_table", torch.int32, (None,))
    dev = q.device
    _pos_tensor(d_pos, dev)
    out, lse = _outputs(q_len, hq, d, dev, out, lse, want_lse)
    _on(dev, q=q, k_pool=k_pool, v_pool=v_pool, page_table=page_table)
    dims = _dims(q, hkv, scale)
    L = lib()
    ws, wsb = _workspace(L.verify_attn_paged_workspace_bytes(ctypes.byref(dims), pos_cap + q_len,
                                                             CHUNK, num_splits), dev, workspace)
    check("verify_attn_paged_dev", L.verify_attn_paged_dev(
        ctypes.byref(dims), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(page_table),
        page_table.numel(), n_slots, CHUNK, _ptr(d_pos), pos_cap, num_splits, _ptr(ws), wsb,
        _ptr(out), _ptr(lse), _stream(stream, dev)))
    return out, lse


def _new_rows(q, k_new, v_new, hkv: int):
    """The block's own rows [q_len][Hkv][D] bf16, one per query row of q."""
    n, h, d = _rows_pair(k_new, v_new, "k_new", "v_new")
    if n != q.shape[0] or h != hkv or d != q.shape[2]:
        raise ValueError(f"k_new/v_new are [{n}][{h}][{d}], need [{q.shape[0]}][{hkv}][{q.shape[2]}]"
                         " (the block's rows: one per query)")


def verify_attn_ring_append_dev(q, k_new, v_new, k_ring, v_ring, d_pos, pos_cap: int,
                                window: int, *, num_splits: int = 0, scale: float = 0.0, out=None,
                                lse=None, want_lse: bool = True, workspace=None, stream=None):
    """verify_kv_append_ring_dev(k_new, v_new, ...) then verify_attn_ring_dev(q, ...) in one
    launch: the block's rows are written into the ring and attended."""
    _form(q, "q", torch.bfloat16, (None, None, None))
    q_len, hq, d = q.shape
    n_chunks, hkv, _ = _chunked(k_ring, v_ring, "k_ring", "v_ring", d)
    _new_rows(q, k_new, v_new, hkv)
    dev = q.device
    _pos_tensor(d_pos, dev)
    out, lse = _outputs(q_len, hq, d, dev, out, lse, want_lse)
    _on(dev, q=q, k_new=k_new, v_new=v_new, k_ring=k_ring, v_ring=v_ring)
    ring_size = n_chunks * CHUNK
    dims = _dims(q, hkv, scale)
    L = lib()
    ws, wsb = _ring_workspace(L.verify_attn_ring_workspace_bytes(ctypes.byref(dims), ring_size,
                                                                 window, num_splits), dev, workspace)
    check("verify_attn_ring_append_dev", L.verify_attn_ring_append_dev(
        ctypes.byref(dims), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_ring), _ptr(v_ring),
        _ptr(d_pos), pos_cap, ring_size, window, num_splits, _ptr(ws), wsb, _ptr(out), _ptr(lse),
        _stream(stream, dev)))
    return out, lse


def verify_attn_paged_append_dev(q, k_new, v_new, k_pool, v_pool, page_table, d_pos,
                                 pos_cap: int, *, num_splits: int = 0, scale: float = 0.0,
                                 out=None, lse=None, want_lse: bool = True, workspace=None,
                                 stream=None):
    """verify_kv_append_paged_dev(k_new, v_new, ...) then verify_attn_paged_dev(q, ...) in one
    launch (plus the split merge): the block's rows are written into their pool slots (from
    page_table) and attended."""
    _form(q, "q", torch.bfloat16, (None, None, None))
    q_len, hq, d = q.shape
    n_slots, hkv, _ = _chunked(k_pool, v_pool, "k_pool", "v_pool", d)
    _new_rows(q, k_new, v_new, hkv)
    _form(page_table, "page_table", torch.int32, (None,))
    dev = q.device
    _pos_tensor(d_pos, dev)
    out, lse = _outputs(q_len, hq, d, dev, out, lse, want_lse)
    _on(dev, q=q, k_new=k_new, v_new=v_new, k_pool=k_pool, v_pool=v_pool, page_table=page_table)
    dims = _dims(q, hkv, scale)
    L = lib()
    ws, wsb = _workspace(L.verify_attn_paged_workspace_bytes(ctypes.byref(dims), pos_cap + q_len,
                                                             CHUNK, num_splits), dev, workspace)
    check("verify_attn_paged_append_dev", L.verify_attn_paged_append_dev(
        ctypes.byref(dims), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_pool), _ptr(v_pool),
        _ptr(page_table), page_table.numel(), n_slots, CHUNK, _ptr(d_pos), pos_cap, num_splits,
        _ptr(ws), wsb, _ptr(out), _ptr(lse), _stream(stream, dev)))
    return out, lse


def verify_kv_append_ring_dev(k_new, v_new, d_pos, pos_cap: int, k_ring, v_ring, *, stream=None):
    """Append rows k_new, v_new [n][Hkv][D] at positions *d_pos .. (device-resident) to the ring."""
    n, hkv, d = _rows_pair(k_new, v_new, "k_new", "v_new")
    n_chunks, _, _ = _chunked(k_ring, v_ring, "k_ring", "v_ring", d, hkv)
    dev = k_new.device
    _pos_tensor(d_pos, dev)
    _on(dev, k_new=k_new, v_new=v_new, k_ring=k_ring, v_ring=v_ring)
    check("verify_kv_append_ring_dev", lib().verify_kv_append_ring_dev(
        _ptr(k_new), _ptr(v_new), n, _ptr(d_pos), pos_cap, hkv, d, _ptr(k_ring), _ptr(v_ring),
        n_chunks * CHUNK, _stream(stream, dev)))


def verify_kv_append_paged_dev(k_new, v_new, d_pos, pos_cap: int, k_pool, v_pool, page_table, *,
                               stream=None):
    """Append rows at positions *d_pos .. to the pool, each chunk's slot read from page_table
    (reserved by the caller for every chunk up to position pos_cap + n - 1)."""
    n, hkv, d = _rows_pair(k_new, v_new, "k_new", "v_new")
    n_slots, _, _ = _chunked(k_pool, v_pool, "k_pool", "v_pool", d, hkv)
    _form(page_table, "page_table", torch.int32, (None,))
    dev = k_new.device
    _pos_tensor(d_pos, dev)
    _on(dev, k_new=k_new, v_new=v_new, k_pool=k_pool, v_pool=v_pool, page_table=page_table)
    check("verify_kv_append_paged_dev", lib().verify_kv_append_paged_dev(
        _ptr(k_new), _ptr(v_new), n, _ptr(d_pos), pos_cap, hkv, d, _ptr(k_pool), _ptr(v_pool),
        _ptr(page_table), page_table.numel(), n_slots, _stream(stream, dev)))


def verify_pos_advance(d_pos, accept_len, *, stream=None):
    """*d_pos += *accept_len + 1 on the device (the tokens one decode step committed)."""
    dev = d_pos.device
    _pos_tensor(d_pos, dev)
    _form(accept_len, "accept_len", torch.int32, (1,))
    _on(dev, accept_len=accept_len)
    check("verify_pos_advance", lib().verify_pos_advance(_ptr(d_pos), _ptr(accept_len),
                                                         _stream(stream, dev)))


def tensor_from_numpy(arr, device="cuda", bf16_bits: Optional[bool] = None) -> torch.Tensor:
    """Copy a numpy array to the device; uint16 arrays are bf16 bit patterns."""
    import numpy as np
    a = np.ascontiguousarray(arr)
    if bf16_bits is None:
        bf16_bits = a.dtype == np.uint16
    if bf16_bits:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(a).to(device)
