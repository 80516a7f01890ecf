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
