"""Pins of the cache oracle (appending a verify block's rows, committing the accepted ones):
over whole decode sequences, attention read from the ring and the pool after every append /
commit equals contiguous attention over the true history (the committed rows plus the current
block's), whose own pins tie it to a library routine; plus the slot bookkeeping's invariants
(CPU only)."""
import numpy as np
import pytest

import oracle
from synth import round_f32_to_bf16_bits

CH = 64


def _bits(g, shape):
    return round_f32_to_bf16_bits(g.standard_normal(shape).astype(np.float32))


def _decode_sequence(seed, steps, q_len, hq, hkv, d, ring, window, n_slots, prefill):
    """Runs `steps` verify blocks; yields (what, got, want) per block and store."""
    g = np.random.default_rng(seed)
    n_table = n_slots
    kr = _bits(g, (ring // CH, hkv, CH, d))            # arbitrary junk before anything is written
    vr = _bits(g, (ring // CH, hkv, d, CH))
    kp = _bits(g, (n_slots, hkv, CH, d))
    vp = _bits(g, (n_slots, hkv, d, CH))
    pager = oracle.PagerModel(n_slots, n_table)
    hist_k = np.zeros((0, hkv, d), np.uint16)
    hist_v = np.zeros((0, hkv, d), np.uint16)
    ctx = 0
    # prefill in blocks, all committed
    while ctx < prefill:
        n = min(q_len * 4, prefill - ctx)
        kb, vb = _bits(g, (n, hkv, d)), _bits(g, (n, hkv, d))
        kr, vr = oracle.append_ring(kr, vr, kb, vb, ctx)
        pager.reserve(n)
        kp, vp = oracle.append_paged(kp, vp, pager.table, kb, vb, ctx)
        pager.commit(n)
        hist_k, hist_v = np.concatenate([hist_k, kb]), np.concatenate([hist_v, vb])
        ctx += n
    for _ in range(steps):
        kb, vb = _bits(g, (q_len, hkv, d)), _bits(g, (q_len, hkv, d))
        q = _bits(g, (q_len, hq, d))
        kr, vr = oracle.append_ring(kr, vr, kb, vb, ctx)
        pager.reserve(q_len)
        kp, vp = oracle.append_paged(kp, vp, pager.table, kb, vb, ctx)
        rows_k, rows_v = np.concatenate([hist_k, kb]), np.concatenate([hist_v, vb])
        total = ctx + q_len
        want_w = oracle.attention_contiguous(q, rows_k, rows_v, total, window=window, dtype="bf16")
        got_w = oracle.attention_ring(q, kr, vr, ctx, ctx % ring, ring, window)
        yield "ring", got_w, want_w
        want_f = oracle.attention_contiguous(q, rows_k, rows_v, total, dtype="bf16")
        got_f = oracle.attention_paged(q, kp, vp, np.array(pager.table), total)
        yield "pool", got_f, want_f
        keep = int(g.integers(1, q_len + 1))          # accepted drafts + the block's first row
        pager.commit(keep)
        hist_k, hist_v = np.concatenate([hist_k, kb[:keep]]), np.concatenate([hist_v, vb[:keep]])
        ctx += keep


def sequence_matches(seed, q_len, ring, window, prefill, steps=12):
    """True when every block of a decode sequence reads the true history from both stores (a
    table that points nowhere, which a wrong rule can leave, counts as a mismatch)."""
    try:
        for _, got, want in _decode_sequence(seed, steps, q_len, 4, 2, 64, ring, window, 16,
                                             prefill):
            if not (np.abs(got[0] - want[0]).max() <= 1e-12 and
                    np.all(np.abs(got[1] - want[1]) <= 1e-12)):
                return False
    except (ValueError, IndexError):
        return False
    return True


@pytest.mark.parametrize("seed,q_len,ring,window,prefill", [
    (1, 16, 256, 100, 150),      # ring wraps within a few blocks; pool chunks freed and reused
    (2, 8, 128, 121, 121),       # window + q_len - 1 == ring size
    (3, 5, 192, 64, 0),          # from an empty context
])
def test_attention_after_appends_equals_contiguous(seed, q_len, ring, window, prefill):
    n = 0
    for what, got, want in _decode_sequence(seed, 12, q_len, 4, 2, 64, ring, window, 16, prefill):
        np.testing.assert_allclose(got[0], want[0], rtol=0, atol=1e-12, err_msg=what)
        np.testing.assert_allclose(got[1], want[1], rtol=0, atol=1e-12, err_msg=what)
        n += 1
    assert n == 24


def test_rejected_rows_would_be_visible_if_not_overwritten():
    # the pin is not vacuous: skipping the next append leaves rejected rows in the ring, and the
    # ring read then differs from the true history
    g = np.random.default_rng(7)
    hkv, d, ring, w, q_len = 1, 64, 128, 64, 8
    kr = np.zeros((ring // CH, hkv, CH, d), np.uint16)
    vr = np.zeros((ring // CH, hkv, d, CH), np.uint16)
    rows_k, rows_v = _bits(g, (40, hkv, d)), _bits(g, (40, hkv, d))
    kr, vr = oracle.append_ring(kr, vr, rows_k, rows_v, 0)
    # block at 40..47, only 2 kept; a shorter next query block (1 row at 42) without its append
    kb, vb = _bits(g, (q_len, hkv, d)), _bits(g, (q_len, hkv, d))
    kr, vr = oracle.append_ring(kr, vr, kb, vb, 40)
    q = _bits(g, (1, 1, d))
    hist_k = np.concatenate([rows_k, kb[:2]])
    hist_v = np.concatenate([rows_v, vb[:2]])
    true = oracle.attention_contiguous(q, hist_k, hist_v, 42, window=w, dtype="bf16")
    stale = oracle.attention_ring(q, kr, vr, 41, 41 % ring, ring, w)    # query at 41 sees 0..41
    np.testing.assert_allclose(stale[0], true[0], atol=1e-12)          # rows <= 41 are committed
    ext = oracle.attention_ring(q, kr, vr, 43, 43 % ring, ring, w)      # a query at 43 would see
    ref = oracle.attention_contiguous(q, np.concatenate([hist_k, kb[2:4]]),   # the stale rows
                                      np.concatenate([hist_v, vb[2:4]]), 44, window=w, dtype="bf16")
    np.testing.assert_allclose(ext[0], ref[0], atol=1e-12)


def test_append_ring_wraps_at_the_ring_size():
    # positions R-2 .. R+1 land in slots R-2, R-1, 0, 1
    hkv, d, ring = 1, 64, 128
    k = np.zeros((ring // CH, hkv, CH, d), np.uint16)
    v = np.zeros((ring // CH, hkv, d, CH), np.uint16)
    kb = np.arange(4 * d, dtype=np.uint16).reshape(4, 1, d) + 1
    k2, v2 = oracle.append_ring(k, v, kb, kb, ring - 2)
    assert np.array_equal(k2[1, 0, 62], kb[0, 0]) and np.array_equal(k2[1, 0, 63], kb[1, 0])
    assert np.array_equal(k2[0, 0, 0], kb[2, 0]) and np.array_equal(k2[0, 0, 1], kb[3, 0])
    assert np.array_equal(v2[0, 0, :, 1], kb[3, 0])
    assert np.count_nonzero(k2) == np.count_nonzero(kb)
    assert np.count_nonzero(k) == 0                     # inputs are not modified


def test_pager_model_invariants_random():
    g = np.random.default_rng(11)
    n_slots, n_table = 12, 40
    p = oracle.PagerModel(n_slots, n_table)
    for step in range(400):
        n = int(g.integers(1, 150))
        try:
            first, slots = p.reserve(n)
        except MemoryError:
            # exhausted: nothing changed; a smaller block may still fit
            assert p.pending is None
            continue
        assert first == -(-p.ctx // CH)
        assert len(slots) == -(-(p.ctx + n) // CH) - first
        keep = int(g.integers(0, n + 1))
        p.commit(keep)
        used = [s for s in p.table if s >= 0]
        assert len(used) == len(set(used))                          # no slot twice
        assert len(used) + len(p.free) == n_slots                    # nothing lost
        assert sorted(used + p.free) == list(range(n_slots))
        nc = -(-p.ctx // CH)
        assert all(s >= 0 for s in p.table[:nc])                     # committed chunks mapped
        assert all(s == -1 for s in p.table[nc:])                    # nothing past them
        if len(used) == n_slots:
            break


def test_pager_model_policy_and_errors():
    p = oracle.PagerModel(4, 8)
    assert p.reserve(130) == (0, [0, 1, 2])
    p.commit(64)                                         # chunks 1, 2 freed: 2 first, then 1
    assert p.table[:3] == [0, -1, -1] and p.free == [3, 2, 1]
    assert p.reserve(10) == (1, [1])                     # the earliest freed chunk's slot first
    with pytest.raises(ValueError):
        p.reserve(1)                                     # a block is pending
    p.commit(0)
    assert p.ctx == 64 and p.table[1] == -1
    with pytest.raises(ValueError):
        p.commit(1)                                      # nothing pending
    with pytest.raises(MemoryError):
        p.reserve(1000)                                  # table has 8 chunks, 1 used
    assert p.pending is None and p.ctx == 64


# --- host paging and the resident subset -----------------------------------------------------

def _pool_case(seed, ctx, hkv=2, d=16, n_slots=None, q_len=16, hq=4):
    from synth import paged_case
    return paged_case(seed, 0, ctx, q_len, hq, hkv, d, n_slots=n_slots)


def test_page_out_in_round_trip_is_bit_exact():
    c = _pool_case(41, 1000, n_slots=24)
    nch = -(-1000 // CH)
    kh = np.zeros((nch,) + c.k_pool.shape[1:], np.uint16)
    vh = np.zeros((nch,) + c.v_pool.shape[1:], np.uint16)
    ids = [3, 5, 6, 0]
    slots = [int(c.page_table[i]) for i in ids]
    kh, vh = oracle.page_out(c.k_pool, c.v_pool, slots, ids, kh, vh)
    for i, s in zip(ids, slots):
        np.testing.assert_array_equal(kh[i], c.k_pool[s])
        np.testing.assert_array_equal(vh[i], c.v_pool[s])
    assert not np.any(kh[[1, 2, 4]])                      # other entries untouched
    # back into other slots: the same bits at the new places, and the same attention
    free = [s for s in range(24) if s not in set(c.page_table.tolist())]
    new = free[:4]
    kp, vp = oracle.page_in(kh, vh, ids, new, c.k_pool, c.v_pool)
    for s_old, s_new in zip(slots, new):
        np.testing.assert_array_equal(kp[s_new], c.k_pool[s_old])
        np.testing.assert_array_equal(vp[s_new], c.v_pool[s_old])
    pt = c.page_table.copy()
    pt[ids] = new
    a = oracle.attention_paged(c.q, c.k_pool, c.v_pool, c.page_table, 1000)
    b = oracle.attention_paged(c.q, kp, vp, pt, 1000)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


def test_resident_all_chunks_equals_paged():
    c = _pool_case(42, 1500)
    ids = list(range(-(-1500 // CH)))
    got = oracle.attention_resident(c.q, c.k_pool, c.v_pool, ids, c.page_table[ids].tolist(), 1500)
    want = oracle.attention_paged(c.q, c.k_pool, c.v_pool, c.page_table, 1500)
    np.testing.assert_array_equal(got[0], want[0])
    np.testing.assert_array_equal(got[1], want[1])


@pytest.mark.parametrize("ctx,q_len,keep", [(1500, 16, (0, 3, 7, 8, 20, 21, 22, 23)),
                                           (3000, 200, (1, 2, 10, 40, 43, 44, 45, 46)),
                                           (640, 70, (8, 9))])
def test_resident_subset_matches_sdpa_with_mask(ctx, q_len, keep):
    import torch
    c = _pool_case(43, ctx, q_len=q_len)
    ids = list(keep)
    got = oracle.attention_resident(c.q, c.k_pool, c.v_pool, ids, c.page_table[ids].tolist(), ctx)
    # library routine over the contiguous rows, keys limited to the resident chunks
    G = 2
    q = torch.from_numpy(oracle.bf16_to_f64(c.q)).permute(1, 0, 2)[None]
    k = torch.from_numpy(oracle.bf16_to_f64(c.k_rows)).permute(1, 0, 2).repeat_interleave(G, 0)[None]
    v = torch.from_numpy(oracle.bf16_to_f64(c.v_rows)).permute(1, 0, 2).repeat_interleave(G, 0)[None]
    qp = torch.arange(ctx - q_len, ctx)[:, None]
    kp = torch.arange(ctx)[None, :]
    mask = (kp <= qp) & torch.isin(kp // CH, torch.tensor(ids))
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask)
    np.testing.assert_allclose(got[0], ref[0].permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)


@pytest.mark.parametrize("ctx,q_len,keep", [(1500, 16, (0, 3, 7, 23)),
                                           (3000, 200, (2, 10, 43, 44, 45, 46)),
                                           (4096, 64, (5, 63))])
def test_resident_equals_packed_pool_at_a_shorter_context(ctx, q_len, keep):
    # the reading the library's resident call uses: with the block's chunks at the end of the
    # list, every earlier resident chunk is wholly visible, so the attention equals attention
    # over the packed slot list at ctx - 64 * (chunks missing before the block's first chunk)
    c = _pool_case(44, ctx, q_len=q_len)
    ids = list(keep)
    slots = c.page_table[ids].tolist()
    got = oracle.attention_resident(c.q, c.k_pool, c.v_pool, ids, slots, ctx)
    first = (ctx - q_len) // CH
    missing = first - ids.index(first)
    virt = oracle.attention_paged(c.q, c.k_pool, c.v_pool, np.array(slots), ctx - CH * missing)
    np.testing.assert_allclose(got[0], virt[0], rtol=0, atol=1e-14)
    np.testing.assert_allclose(got[1], virt[1], rtol=0, atol=1e-13)


def test_pager_model_evict_restore_policy_and_errors():
    p = oracle.PagerModel(6, 10)
    p.reserve(200)                                       # chunks 0..3 -> slots 0..3
    p.commit(200)                                        # ctx 200: chunks 0, 1, 2 full, 3 partial
    assert p.evict([1, 0]) == [1, 0]
    assert p.table[:4] == [oracle.PAGED_OUT, oracle.PAGED_OUT, 2, 3] and p.free[-2:] == [1, 0]
    assert p.resident() == ([2, 3], [2, 3])
    for bad in ([3], [0], [2, 2], [-1], [7]):            # partial tail, already out, twice, range
        with pytest.raises(ValueError):
            p.evict(bad)
    assert p.restore([1]) == [0]                         # the last freed slot first
    with pytest.raises(ValueError):
        p.restore([2])                                   # resident
    p.reserve(100)                                       # a block while chunk 0 is out
    assert p.resident()[0] == [1, 2, 3, 4]
    with pytest.raises(ValueError):
        p.evict([3])                                     # the chunk the pending block writes
    p.commit(100)                                        # ctx 300: chunks 0..3 full
    assert p.evict([3, 2]) == [3, 2]
    assert p.restore([0, 2, 3]) == [2, 3, 4]
    # not enough free slots: nothing changes
    q = oracle.PagerModel(2, 4)
    q.reserve(128)
    q.commit(128)
    q.evict([0, 1])
    q.reserve(64)
    q.commit(64)
    before = (list(q.table), list(q.free))
    with pytest.raises(MemoryError):
        q.restore([0, 1])
    assert (q.table, q.free) == before


def test_pager_model_paging_invariants_random():
    g = np.random.default_rng(45)
    p = oracle.PagerModel(20, 80)
    for _ in range(300):
        op = g.integers(0, 3)
        if op == 0:
            n = int(g.integers(1, 200))
            try:
                p.reserve(n)
            except MemoryError:
                continue
            p.commit(int(g.integers(0, n + 1)))
        elif op == 1:
            full = p.ctx // CH
            cand = [c for c in range(full) if p.table[c] >= 0]
            if cand:
                pick = list(g.choice(cand, size=min(len(cand), int(g.integers(1, 4))), replace=False))
                p.evict([int(c) for c in pick])
        else:
            out = [c for c, s in enumerate(p.table) if s == oracle.PAGED_OUT]
            if out:
                pick = [int(c) for c in g.choice(out, size=min(len(out), 2), replace=False)]
                try:
                    p.restore(pick)
                except MemoryError:
                    pass
        used = [s for s in p.table if s >= 0]
        assert len(used) == len(set(used))
        assert sorted(used + p.free) == list(range(20))
        nc = -(-p.ctx // CH)
        assert all(s != -1 for s in p.table[:nc])             # committed: resident or paged out
        assert all(s == -1 for s in p.table[nc:])
        ids, slots = p.resident()
        assert ids == sorted(ids) and all(p.table[c] == s for c, s in zip(ids, slots))
