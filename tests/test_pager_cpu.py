"""The library's host-side pager (rkv_pager_*, through the C interface, no GPU) against the
oracle's slot bookkeeping: same tables, same slots, same free counts and the same refusals over
random reserve / commit sequences; plus its argument checks."""
import ctypes
import os

import numpy as np
import pytest

import oracle
from ring_kv_amd import _lib

if not os.path.exists(_lib.LIB_PATH):
    pytest.skip("libring_kv.so not built (run python -m ring_kv_amd.build)", allow_module_level=True)

import ring_kv_amd as rk  # noqa: E402

L = _lib.lib()
OK, ENULL, ETABLE, EARG = 0, -1, -5, -8


@pytest.mark.parametrize("seed,n_slots,n_table,max_n", [(1, 12, 40, 150), (2, 64, 64, 1024),
                                                        (3, 3, 1000, 200), (4, 200, 100, 70)])
def test_pager_matches_model(seed, n_slots, n_table, max_n):
    g = np.random.default_rng(seed)
    p, m = rk.Pager(n_slots, n_table), oracle.PagerModel(n_slots, n_table)
    refused = 0
    for _ in range(500):
        n = int(g.integers(1, max_n + 1))
        try:
            want = m.reserve(n)
        except MemoryError:
            want = None
        if want is None:
            with pytest.raises(_lib.RkvError) as e:
                p.reserve(n)
            assert e.value.status == ETABLE
            refused += 1
            continue
        assert p.reserve(n) == want
        keep = int(g.integers(0, n + 1))
        m.commit(keep)
        p.commit(keep)
        assert p.ctx_len == m.ctx
        assert p.free_slots == len(m.free)
        assert p.table() == m.table
    p.close()


def test_pager_argument_checks():
    assert not L.rkv_pager_create(0, 10) and not L.rkv_pager_create(10, 0)
    h = L.rkv_pager_create(4, 8)
    first, k = ctypes.c_int32(), ctypes.c_int32()
    slots = (ctypes.c_int32 * 17)()
    assert L.rkv_pager_reserve(None, 10, ctypes.byref(first), ctypes.byref(k), slots) == ENULL
    assert L.rkv_pager_reserve(h, 10, None, ctypes.byref(k), slots) == ENULL
    assert L.rkv_pager_reserve(h, 0, ctypes.byref(first), ctypes.byref(k), slots) == EARG
    assert L.rkv_pager_reserve(h, 1025, ctypes.byref(first), ctypes.byref(k), slots) == EARG
    assert L.rkv_pager_commit(h, 1) == EARG                    # nothing pending
    assert L.rkv_pager_reserve(h, 600, ctypes.byref(first), ctypes.byref(k), slots) == ETABLE
    assert L.rkv_pager_free_slots(h) == 4 and L.rkv_pager_ctx_len(h) == 0   # nothing changed
    assert L.rkv_pager_reserve(h, 100, ctypes.byref(first), ctypes.byref(k), slots) == OK
    assert (first.value, k.value, slots[0], slots[1]) == (0, 2, 0, 1)
    assert L.rkv_pager_reserve(h, 1, ctypes.byref(first), ctypes.byref(k), slots) == EARG
    assert L.rkv_pager_commit(h, 101) == EARG                  # more than the block
    assert L.rkv_pager_commit(h, 100) == OK
    out = (ctypes.c_int32 * 8)()
    assert L.rkv_pager_table(h, out, 9) == EARG
    assert L.rkv_pager_table(h, out, 8) == OK and list(out) == [0, 1, -1, -1, -1, -1, -1, -1]
    assert L.rkv_pager_ctx_len(None) == -1 and L.rkv_pager_free_slots(None) == -1
    L.rkv_pager_destroy(h)
    L.rkv_pager_destroy(None)


@pytest.mark.parametrize("seed,n_slots,n_table", [(5, 20, 80), (6, 8, 300), (7, 64, 64)])
def test_pager_paging_matches_model(seed, n_slots, n_table):
    """Random reserve / commit / evict / restore sequences: same slots, tables, free counts,
    resident lists and refusals as the oracle's model."""
    g = np.random.default_rng(seed)
    p, m = rk.Pager(n_slots, n_table), oracle.PagerModel(n_slots, n_table)
    for _ in range(600):
        op = int(g.integers(0, 4))
        if op == 0:
            n = int(g.integers(1, 200))
            try:
                want = m.reserve(n)
            except MemoryError:
                with pytest.raises(_lib.RkvError):
                    p.reserve(n)
                continue
            assert p.reserve(n) == want
            keep = int(g.integers(0, n + 1))
            m.commit(keep)
            p.commit(keep)
        elif op in (1, 2):
            # evict: usually valid whole committed chunks, sometimes a chunk that does not qualify
            full = m.ctx // 64
            cand = [c for c in range(full) if m.table[c] >= 0]
            if op == 2 or not cand:
                bad = [int(g.integers(0, n_table))]
                try:
                    m.evict(bad)
                except ValueError:
                    with pytest.raises(_lib.RkvError) as e:
                        p.evict(bad)
                    assert e.value.status == EARG
                    continue
                assert p.evict(bad) is not None
                continue
            pick = [int(c) for c in g.choice(cand, size=min(len(cand), int(g.integers(1, 5))),
                                             replace=False)]
            assert p.evict(pick) == m.evict(pick)
        else:
            out = [c for c, s in enumerate(m.table) if s == oracle.PAGED_OUT]
            if not out:
                continue
            pick = [int(c) for c in g.choice(out, size=min(len(out), int(g.integers(1, 6))),
                                             replace=False)]
            try:
                want = m.restore(pick)
            except MemoryError:
                with pytest.raises(_lib.RkvError) as e:
                    p.restore(pick)
                assert e.value.status == ETABLE
                continue
            assert p.restore(pick) == want
        assert p.table() == m.table
        assert p.free_slots == len(m.free)
        assert p.resident() == m.resident()
    p.close()


def test_pager_paging_argument_checks():
    h = L.rkv_pager_create(4, 8)
    first, k = ctypes.c_int32(), ctypes.c_int32()
    slots = (ctypes.c_int32 * 17)()
    L.rkv_pager_reserve(h, 200, ctypes.byref(first), ctypes.byref(k), slots)
    L.rkv_pager_commit(h, 200)                                 # chunks 0..2 full, 3 partial
    ids = (ctypes.c_int32 * 4)(3, 0, 0, 0)
    out = (ctypes.c_int32 * 4)()
    assert L.rkv_pager_evict(h, ids, 1, out) == EARG           # the partial tail chunk
    ids[0] = 1
    assert L.rkv_pager_evict(h, ids, 2, out) == OK and list(out)[:2] == [1, 0]
    assert L.rkv_pager_evict(h, ids, 1, out) == EARG           # already out
    ids[0], ids[1] = 2, 2
    assert L.rkv_pager_evict(h, ids, 2, out) == EARG           # repeated
    assert L.rkv_pager_evict(None, ids, 1, out) == ENULL
    assert L.rkv_pager_evict(h, None, 1, out) == ENULL
    assert L.rkv_pager_evict(h, ids, -1, out) == EARG
    assert L.rkv_pager_evict(h, None, 0, None) == OK           # nothing to do
    ids[0], ids[1] = 1, 0
    assert L.rkv_pager_restore(h, ids, 2, out) == OK and list(out)[:2] == [0, 1]
    assert L.rkv_pager_restore(h, ids, 1, out) == EARG         # resident
    tab = (ctypes.c_int32 * 8)()
    L.rkv_pager_table(h, tab, 8)
    assert list(tab) == [1, 0, 2, 3, -1, -1, -1, -1]
    assert L.rkv_pager_resident(h, None, None, 0) == 4
    assert L.rkv_pager_resident(h, None, out, 2) == ENULL
    assert L.rkv_pager_resident(None, None, None, 0) == ENULL
    L.rkv_pager_destroy(h)
