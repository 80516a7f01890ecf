"""The torch binding's argument checks (CPU).  The library trusts the sizes it is handed, so the
binding compares every buffer with the sizes the call will use before anything reaches it: a
mismatch names the argument, and arguments that agree get as far as the device check (host
tensors here), never to the library."""
import pytest
import torch

import ring_kv_amd as rk

bf, f32, i32 = torch.bfloat16, torch.float32, torch.int32


def z(*shape, dtype=bf):
    return torch.zeros(shape, dtype=dtype)


def _fails(fn, *words):
    with pytest.raises((ValueError, TypeError)) as e:
        fn()
    msg = str(e.value)
    assert all(w in msg for w in words), msg


def _reaches_device_check(fn):
    _fails(fn, "must be a device tensor")


Q = z(16, 16, 128)
KP, VP = z(40, 4, 64, 128), z(40, 4, 128, 64)
PT = z(40, dtype=i32)


def test_paged_checks():
    _reaches_device_check(lambda: rk.verify_attn_paged(Q, KP, VP, PT, 2000))
    _fails(lambda: rk.verify_attn_paged(z(16, 16, 64), KP, VP, PT, 2000), "k_pool", "[*][*][64][64]")
    _fails(lambda: rk.verify_attn_paged(Q, KP, z(40, 4, 64, 128), PT, 2000), "v_pool")
    _fails(lambda: rk.verify_attn_paged(Q, z(40, 4, 32, 128), VP, PT, 2000), "k_pool")
    _fails(lambda: rk.verify_attn_paged(Q, KP, z(41, 4, 128, 64), PT, 2000), "v_pool")
    _fails(lambda: rk.verify_attn_paged(Q, KP, VP, z(40), 2000), "page_table", "dtype")
    _fails(lambda: rk.verify_attn_paged(Q, KP, VP, PT, 2000, out=z(16, 16, 64, dtype=f32)), "out")
    _fails(lambda: rk.verify_attn_paged(Q, KP, VP, PT, 2000, lse=z(16, 8, dtype=f32)), "lse")
    _fails(lambda: rk.verify_attn_paged(Q, KP, VP, PT, 2000, out=z(16, 16, 128)), "out", "dtype")
    _fails(lambda: rk.verify_attn_paged(Q.transpose(0, 1), KP, VP, PT, 2000), "contiguous")
    _fails(lambda: rk.verify_attn_paged(3, KP, VP, PT, 2000), "torch.Tensor")


def test_partial_and_merge_checks():
    _reaches_device_check(lambda: rk.verify_attn_paged_partial(Q, KP, VP, PT, 2000, 8))
    _fails(lambda: rk.verify_attn_paged_partial(Q, KP, VP, PT, 2000, 8,
                                                part_out=z(4, 8, 32, 128, dtype=f32)), "part_out")
    _fails(lambda: rk.verify_attn_paged_partial(Q, KP, VP, PT, 2000, 8,
                                                part_lse=z(4, 7, 64, dtype=f32)), "part_lse")
    _fails(lambda: rk.verify_attn_paged_partial(Q, KP, VP, PT, 2000, 0), "num_splits")
    po, pl = z(4, 8, 64, 128, dtype=f32), z(4, 8, 64, dtype=f32)
    _reaches_device_check(lambda: rk.attn_merge_partials(po, pl, 16, 16))
    _fails(lambda: rk.attn_merge_partials(po, pl, 8, 16), "rows")
    _fails(lambda: rk.attn_merge_partials(po, pl, 16, 18), "rows")
    _fails(lambda: rk.attn_merge_partials(po, z(4, 8, 63, dtype=f32), 16, 16), "part_lse")
    _fails(lambda: rk.attn_merge_partials(po, pl, 16, 16, out=z(16, 16, 64, dtype=f32)), "out")


def test_ring_and_contiguous_checks():
    KR, VR = z(32, 4, 64, 128), z(32, 4, 128, 64)
    _reaches_device_check(lambda: rk.verify_attn_ring(Q, KR, VR, 30000, 512))
    _fails(lambda: rk.verify_attn_ring(Q, KR, z(32, 4, 64, 128), 30000, 512), "v_ring")
    _fails(lambda: rk.verify_attn_ring(z(16, 16, 64), KR, VR, 30000, 512), "k_ring")
    q = z(16, 8, 64, dtype=f32)
    k = z(1024, 2, 64, dtype=f32)
    _reaches_device_check(lambda: rk.decode_attn_ref_layout(q, k, k.clone(), 1024))
    _fails(lambda: rk.decode_attn_ref_layout(q, z(1024, 2, 32, dtype=f32), k, 1024), "k")
    _fails(lambda: rk.decode_attn_ref_layout(q, k, z(1000, 2, 64, dtype=f32), 1000), "v")
    _fails(lambda: rk.decode_attn_ref_layout(q, k, k.clone(), 1025), "fewer than ctx_len")
    _fails(lambda: rk.decode_attn_ref_layout(q, k.to(bf), k.to(bf), 1024), "k", "dtype")


def test_accept_checks():
    L, P = z(17, 4096, dtype=f32), z(16, dtype=i32)
    _reaches_device_check(lambda: rk.verify_accept(L, P))
    _fails(lambda: rk.verify_accept(z(16, 4096, dtype=f32), P), "logits")
    _fails(lambda: rk.verify_accept(L, P, committed=z(16, dtype=i32)), "committed")
    _fails(lambda: rk.verify_accept(L, P, row_argmax=z(18, dtype=i32)), "row_argmax")
    _fails(lambda: rk.verify_accept(L, P, accept_len=z(0, dtype=i32)), "accept_len")
    _fails(lambda: rk.verify_accept(L, z(16, dtype=torch.int64)), "proposals", "dtype")


def test_layout_and_append_checks():
    kr, vr = z(32, 4, 64, 128), z(32, 4, 128, 64)
    rows = z(100, 4, 128)
    _reaches_device_check(lambda: rk.ref_layout_to_ring(rows, rows.clone(), 0, kr, vr))
    _fails(lambda: rk.ref_layout_to_ring(rows, z(100, 4, 64), 0, kr, vr), "v_src")
    _fails(lambda: rk.ref_layout_to_ring(z(100, 2, 128), z(100, 2, 128), 0, kr, vr), "k_ring")
    _reaches_device_check(lambda: rk.ref_layout_to_paged(rows, rows.clone(), 0, KP, VP, PT))
    _fails(lambda: rk.ref_layout_to_paged(rows, rows.clone(), 0, KP, z(40, 4, 64, 128), PT),
           "v_pool")
    blk = z(16, 4, 128)
    _reaches_device_check(lambda: rk.verify_kv_append_ring(blk, blk.clone(), 0, kr, vr))
    _fails(lambda: rk.verify_kv_append_ring(blk, z(16, 4, 64), 0, kr, vr), "v_new")
    _reaches_device_check(lambda: rk.verify_kv_append_paged(blk, blk.clone(), 0, KP, VP, PT, 0, [3]))
    _fails(lambda: rk.verify_kv_append_paged(z(16, 4, 64), z(16, 4, 64), 0, KP, VP, PT, 0, [3]),
           "k_pool")


def test_paging_and_resident_checks():
    kh, vh = z(100, 4, 64, 128), z(100, 4, 128, 64)
    _reaches_device_check(lambda: rk.kv_page_out(KP, VP, [1], [7], kh, vh))
    _fails(lambda: rk.kv_page_out(KP, VP, [1], [7], z(100, 4, 64, 64), vh), "k_host")
    _fails(lambda: rk.kv_page_out(KP, VP, [1], [7], kh, z(100, 2, 128, 64)), "v_host")
    _fails(lambda: rk.kv_page_in(kh, z(99, 4, 128, 64), [7], [1], KP, VP), "v_host")
    _fails(lambda: rk.kv_page_out(KP, VP, [1], [7], kh, vh.to(f32)), "v_host", "dtype")
    ds = z(5, dtype=i32)
    _reaches_device_check(lambda: rk.verify_attn_paged_resident(Q, KP, VP, ds, [0, 1, 2, 3, 4], 320))
    _fails(lambda: rk.verify_attn_paged_resident(Q, KP, VP, ds, [0, 1, 2, 3], 256), "d_slots")
    _fails(lambda: rk.verify_attn_paged_resident(Q, KP, VP, ds, [0, 1, 2, 3, 4], 320,
                                                 lse=z(16, 16, 1, dtype=f32)), "lse")


def test_ring_counter_bytes_match_the_header():
    """The binding sizes its own ring workspaces without the counters the header reserves at the
    start of a full-size one (so a fresh workspace needs no zeroing); both must name the same
    size."""
    import os
    import re
    hdr = open(os.path.join(os.path.dirname(__file__), "..", "include", "ring_kv.h")).read()
    m = re.search(r"#define RKV_RING_COUNTER_BYTES (\d+)", hdr)
    assert m and int(m.group(1)) == rk.api.RING_COUNTER_BYTES
