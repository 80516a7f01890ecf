"""The C library loads without a GPU, exports every function include/ring_kv.h declares, and
rejects bad arguments on the host with the documented status before any HIP call (a call that
reached a launch here, with no GPU, would report RKV_ERR_HIP instead)."""
import ctypes
import os

import pytest

from ring_kv_amd import _lib
from ring_kv_amd._lib import AttnDims

if not os.path.exists(_lib.LIB_PATH):
    pytest.skip("libring_kv.so not built (run python -m ring_kv_amd.build)", allow_module_level=True)

L = _lib.lib()
NULL = None
P = ctypes.c_void_p(0x1000)          # never dereferenced: every call below stops on the host
OK, ENULL, ESHAPE, EDTYPE, ERING, ETABLE, EWS, EHIP, EARG = 0, -1, -2, -3, -4, -5, -6, -7, -8


def dims(q_len=16, hq=16, hkv=4, d=128, scale=0.0, dtype=1):
    return ctypes.byref(AttnDims(q_len, hq, hkv, d, scale, dtype))


def test_exports_every_declared_function():
    names = _lib.declared_functions()
    assert len(names) >= 15
    for n in names:
        assert hasattr(L, n), n
    assert L.rkv_abi_version() == 1
    assert L.rkv_status_str(-6) == b"workspace missing or too small"


def paged(d=None, q=P, k=P, v=P, pt=P, n_table=4096, n_slots=4096, chunk=64, ctx=262144,
          splits=0, ws=P, wsb=1 << 30, out=P):
    return L.verify_attn_paged(dims() if d is None else d, q, k, v, pt, n_table, n_slots, chunk,
                               ctx, splits, ws, wsb, out, NULL, NULL)


def test_paged_argument_checks():
    assert L.verify_attn_paged(None, P, P, P, P, 4096, 4096, 64, 262144, 0, P, 1 << 30, P, NULL, NULL) == ENULL
    assert paged(q=NULL) == ENULL and paged(pt=NULL) == ENULL and paged(out=NULL) == ENULL
    assert paged(d=dims(d=96)) == ESHAPE
    assert paged(d=dims(hq=10, hkv=4)) == ESHAPE
    assert paged(d=dims(q_len=4097)) == ESHAPE          # 4097 * 4 rows > 16384
    assert paged(d=dims(q_len=0)) == ESHAPE
    assert paged(d=dims(dtype=0)) == EDTYPE               # the chunked stores are bf16
    assert paged(d=dims(dtype=7)) == EDTYPE
    assert paged(d=dims(scale=-1.0)) == EARG
    assert paged(chunk=32) == ETABLE
    assert paged(n_table=4095) == ETABLE
    assert paged(n_slots=0) == ETABLE
    assert paged(ctx=15) == ESHAPE                        # the block must fit in the context
    assert paged(ws=NULL) == EWS
    assert paged(wsb=1000) == EWS
    assert paged(splits=-1) == EARG


def test_split_span_limit():
    # one split may span at most 2^22 chunks (positions are 32-bit offsets inside a split)
    n = (1 << 22) + 1
    assert paged(n_table=n, n_slots=n, ctx=n * 64, splits=1, ws=NULL, wsb=0) == ESHAPE
    assert L.verify_attn_paged_partial(dims(), P, P, P, P, n, n, 64, n * 64, 1, P, P, NULL) == ESHAPE
    assert L.verify_attn_paged_partial(dims(), P, P, P, P, n, n, 64, n * 64, 0, P, P, NULL) == EARG


def test_paged_workspace_and_splits():
    d = dims()
    # 4 KV heads: 64 splits of 64 chunks at 262,144 positions; partials [4][64][64][128] f32
    assert L.verify_attn_paged_auto_splits(d, 262144, 64) == 64
    want = 4 * 64 * 64 * 128 * 4 + 4 * 64 * 64 * 4
    assert L.verify_attn_paged_workspace_bytes(d, 262144, 64, 0) == want
    assert L.verify_attn_paged_workspace_bytes(d, 262144, 64, 1) == 0     # no merge, no partials
    assert L.verify_attn_paged_auto_splits(d, 131072, 64) == 64
    # shorter contexts: fewer, longer splits (a smaller merge), at least n/4 and 32, at most n
    assert L.verify_attn_paged_auto_splits(d, 16384, 64) == 64           # 4 chunks per split
    assert L.verify_attn_paged_auto_splits(d, 12288, 64) == 48
    assert L.verify_attn_paged_auto_splits(d, 8192, 64) == 32            # 4 chunks per split
    assert L.verify_attn_paged_auto_splits(d, 4096, 64) == 32            # 2 chunks per split
    assert L.verify_attn_paged_auto_splits(d, 1024, 64) == 16            # 1 chunk per split
    assert L.verify_attn_paged_auto_splits(d, 65, 64) == 2
    want8k = 4 * 32 * 64 * 128 * 4 + 4 * 32 * 64 * 4
    assert L.verify_attn_paged_workspace_bytes(d, 8192, 64, 0) == want8k
    assert L.verify_attn_paged_workspace_bytes(d, 262144, 32, 0) == 0    # unsupported chunk


def test_prefill_block_splits():
    # a 1024-token block (4096 rows per KV head) runs 256-row tiles over the pool: 4 heads x 16
    # tiles, so 4 splits give one workgroup per compute unit; partials [4][4][4096][128] f32
    d = dims(q_len=1024)
    assert L.verify_attn_paged_auto_splits(d, 9216, 64) == 4
    want = 4 * 4 * 4096 * 128 * 4 + 4 * 4 * 4096 * 4
    assert L.verify_attn_paged_workspace_bytes(d, 9216, 64, 0) == want
    assert L.verify_attn_paged_auto_splits(d, 131072, 64) == 4
    # over the ring the block is not split: no partials
    assert L.verify_attn_ring_workspace_bytes(d, 2048, 512, 0) == 0
    assert L.verify_attn_ring_workspace_bytes(d, 1024, 512, 0) == 0
    # 17..64-query verify blocks: 2..4 row tiles of 64 share the chip
    assert L.verify_attn_paged_auto_splits(dims(q_len=32), 262144, 64) == 32
    # the longest block one call takes
    assert L.verify_attn_paged_auto_splits(dims(q_len=4096), 262144, 64) == 1
    assert L.verify_attn_paged_auto_splits(dims(q_len=4097), 262144, 64) == 0


def ring(d=None, pos0=30000, head=1328, size=2048, window=512, splits=0, ws=P, wsb=1 << 30):
    return L.verify_attn_ring(dims() if d is None else d, P, P, P, pos0, head, size, window,
                              splits, ws, wsb, P, NULL, NULL)


def test_ring_argument_checks():
    assert ring(head=1327) == ERING                        # head must be pos0 mod ring_size
    assert ring(size=2000, head=30000 % 2000) == ERING     # not a multiple of 64
    assert ring(size=512, head=30000 % 512) == ERING       # 512 < window + q_len - 1
    assert ring(window=0) == EARG
    assert ring(pos0=-1, head=0) == EARG
    assert ring(d=dims(dtype=0)) == EDTYPE
    # 527 positions touch at most 10 chunks: one chunk per split by default; 8,192 bytes of
    # counters, then partials [4][10][64][128] + [4][10][64] floats
    part = 4 * 10 * 64 * 128 * 4 + 4 * 10 * 64 * 4
    want = 8192 + part
    assert L.verify_attn_ring_workspace_bytes(dims(), 2048, 512, 0) == want
    assert L.verify_attn_ring_workspace_bytes(dims(), 2048, 512, 10) == want
    assert ring(ws=NULL) == EWS
    assert ring(wsb=8192) == EWS                           # room for the counters only


def test_contiguous_and_merge_checks():
    d = dims(q_len=16, hq=8, hkv=2, d=64, dtype=0)
    assert L.decode_attn_ref_layout(d, P, P, P, 1024, 0, 0, NULL, 0, P, NULL, NULL) == EWS
    assert L.decode_attn_ref_layout(d, P, P, P, 8, 0, 0, P, 1 << 20, P, NULL, NULL) == ESHAPE
    assert L.decode_attn_ref_layout(d, P, P, P, 1024, -1, 0, P, 1 << 20, P, NULL, NULL) == EARG
    assert L.decode_attn_ref_layout(d, NULL, P, P, 1024, 0, 0, P, 1 << 20, P, NULL, NULL) == ENULL
    assert L.attn_merge_partials(dims(), 0, P, P, P, NULL, NULL) == EARG
    assert L.attn_merge_partials(dims(), 4, NULL, P, P, NULL, NULL) == ENULL
    assert L.verify_attn_paged_partial(dims(), P, P, P, P, 128, 128, 64, 8192, 0, P, P, NULL) == EARG


def test_accept_checks():
    need = L.verify_accept_workspace_bytes(16, 65536)
    assert need == 2 * 1280           # 17 rows x 16 parts of 4096 logits, f32 + i32, 256-B aligned
    assert L.verify_accept(NULL, 16, 65536, P, P, P, NULL, P, need, NULL) == ENULL
    assert L.verify_accept(P, 16, 65536, P, P, P, NULL, NULL, 0, NULL) == EWS
    assert L.verify_accept(P, 16, 65536, P, P, P, NULL, P, need - 1, NULL) == EWS
    assert L.verify_accept(P, 256, 10, P, P, P, NULL, P, 1 << 20, NULL) == ESHAPE
    assert L.verify_accept(P, 16, 0, P, P, P, NULL, P, 1 << 20, NULL) == ESHAPE
    assert L.verify_accept(P, 3, 10, NULL, P, P, NULL, P, 1 << 20, NULL) == ENULL


def test_layout_helper_checks():
    assert L.ref_layout_to_ring(P, P, 0, 3000, 4, 128, 1, P, P, 2048, NULL) == ERING
    assert L.ref_layout_to_ring(P, P, 0, 10, 4, 128, 0, P, P, 2048, NULL) == EDTYPE
    assert L.ref_layout_to_paged(P, P, 0, 8193, 4, 128, 1, P, P, P, 128, 128, 64, NULL) == ETABLE
    assert L.ref_layout_to_paged(P, P, 0, 10, 4, 96, 1, P, P, P, 128, 128, 64, NULL) == ESHAPE
    assert L.ref_layout_to_paged(NULL, P, 0, 0, 4, 128, 1, P, P, P, 128, 128, 64, NULL) == OK
    odd = ctypes.c_void_p(0x1008)                 # 8-byte aligned: the row copies move 16 bytes
    assert L.ref_layout_to_ring(odd, P, 0, 10, 4, 128, 1, P, P, 2048, NULL) == EARG
    assert L.ref_layout_to_paged(P, P, 0, 10, 4, 128, 1, odd, P, P, 128, 128, 64, NULL) == EARG
    assert L.verify_kv_append_ring(P, odd, 16, 100, 4, 128, P, P, 2048, NULL) == EARG
    assert L.verify_kv_append_ring_dev(P, P, 16, P, 100, 4, 128, P, odd, 2048, NULL) == EARG


def test_append_checks():
    app_r = lambda n=16, pos=100, hkv=4, d=128, size=2048, k=P: L.verify_kv_append_ring(  # noqa: E731
        k, P, n, pos, hkv, d, P, P, size, NULL)
    assert app_r(k=NULL) == ENULL
    assert app_r(d=96) == ESHAPE and app_r(hkv=0) == ESHAPE
    assert app_r(n=0) == EARG and app_r(n=1025) == EARG and app_r(pos=-1) == EARG
    assert app_r(size=100) == ERING and app_r(n=200, size=128) == ERING
    slots = (ctypes.c_int32 * 2)(5, 6)

    def app_p(n=16, ctx=120, first=2, n_new=1, sl=slots, table=P, n_table=10, n_slots=8):
        return L.verify_kv_append_paged(P, P, n, ctx, 4, 128, P, P, table, n_table, n_slots,
                                        first, n_new, sl, NULL)
    assert app_p(table=NULL) == ENULL and app_p(sl=NULL) == ENULL
    assert app_p(first=1) == EARG                 # ceil(120/64) = 2
    assert app_p(n_new=0) == EARG                 # positions 120..135 start chunk 2
    assert app_p(n=4, n_new=1) == EARG            # 120..123 stay in chunk 1: no new chunk
    assert app_p(ctx=640, first=10, n_new=1) == ETABLE      # past the table
    assert app_p(n_slots=5) == ETABLE                       # slot 5 out of range
    assert app_p(n=0) == EARG and app_p(ctx=-1) == EARG


def _i32(*v):
    return (ctypes.c_int32 * max(1, len(v)))(*v)


def test_page_copy_checks():
    # every case is refused on the host before any HIP call
    ws = L.kv_page_workspace_bytes(4, 128, 3)
    assert ws == 2 * 3 * 4 * 64 * 128 * 2
    assert L.kv_page_workspace_bytes(4, 128, 1000) == 2 * 256 * 4 * 64 * 128 * 2
    assert L.kv_page_workspace_bytes(4, 96, 3) == 0 and L.kv_page_workspace_bytes(4, 128, 0) == 0
    out = lambda sl, ci, n, n_slots=16, n_host=100, wsp=P, wsb=ws, d=128: L.kv_page_out(  # noqa: E731
        P, P, 4, d, n_slots, sl, ci, n, P, P, n_host, wsp, wsb, NULL)
    inn = lambda sl, ci, n, n_slots=16, n_host=100, wsp=P, wsb=ws: L.kv_page_in(  # noqa: E731
        P, P, n_host, ci, sl, n, P, P, 4, 128, n_slots, wsp, wsb, NULL)
    for f in (out, inn):
        assert f(_i32(0, 1, 2), _i32(5, 6, 7), 0) == OK                   # nothing to copy
        assert f(_i32(0, 1, 2), _i32(5, 6, 7), -1) == EARG
        assert f(_i32(0, 1, 16), _i32(5, 6, 7), 3) == ETABLE               # slot past the pool
        assert f(_i32(0, 1, -1), _i32(5, 6, 7), 3) == ETABLE
        assert f(_i32(0, 1, 2), _i32(5, 6, 100), 3) == EARG                # chunk past the store
        assert f(_i32(0, 1, 2), _i32(5, 6, 7), 3, wsp=NULL) == EWS
        assert f(_i32(0, 1, 2), _i32(5, 6, 7), 3, wsb=ws - 1) == EWS
        assert f(NULL, _i32(5, 6, 7), 3) == ENULL
    assert out(_i32(0, 1, 2), _i32(5, 6, 7), 3, d=96) == ESHAPE
    assert out(_i32(0, 1, 2), _i32(5, 5, 7), 3) == EARG                    # one host entry twice
    assert inn(_i32(0, 0, 2), _i32(5, 6, 7), 3) == EARG                    # one slot twice
    assert L.kv_page_out(NULL, P, 4, 128, 16, _i32(0), _i32(0), 1, P, P, 100, P, ws, NULL) == ENULL
    assert L.kv_page_in(P, NULL, 100, _i32(0), _i32(0), 1, P, P, 4, 128, 16, P, ws, NULL) == ENULL


def test_resident_attention_checks():
    # 16-token block at ctx 5000: its positions 4984..4999 lie in chunk 77 (4928..4991) and 78
    res = lambda ids, ctx=5000, d=None: L.verify_attn_paged_resident(  # noqa: E731
        dims() if d is None else d, P, P, P, P, _i32(*ids), len(ids), 160, ctx, 0, P, 1 << 30,
        P, NULL, NULL)
    assert res([]) == ETABLE                                              # nothing resident
    assert res([0, 5, 77]) == ETABLE                                      # chunk 78 missing
    assert res([0, 5, 78]) == ETABLE                                      # chunk 77 missing
    assert res([0, 78, 77]) == ETABLE                                     # not increasing
    assert res([77, 78, 79]) == ETABLE                                    # past the context
    assert res([-1, 77, 78]) == ETABLE
    assert L.verify_attn_paged_resident(dims(), P, P, P, P, None, 2, 160, 5000, 0, P, 1 << 30, P,
                                        NULL, NULL) == ENULL
    assert res([77, 78], ctx=10) == ESHAPE                                # block longer than ctx
    assert res([77, 78], d=dims(d=96)) == ESHAPE
    # valid lists pass the resident checks and meet the paged ones (a null slot list here)
    assert L.verify_attn_paged_resident(dims(), P, P, P, NULL, _i32(3, 77, 78), 3, 160, 5000, 0,
                                        P, 1 << 30, P, NULL, NULL) == ENULL


def test_resident_workspace_is_that_of_its_chunks():
    # the resident call splits the n_res listed chunks like a context of 64 * n_res positions,
    # and split counts are not monotone in the context: 32 chunks take 32 splits of one chunk,
    # more than the 20 of the full 40-chunk context
    d = dims()
    assert L.verify_attn_paged_auto_splits(d, 64 * 32, 64) == 32
    assert L.verify_attn_paged_auto_splits(d, 2560, 64) == 20
    short = L.verify_attn_paged_workspace_bytes(d, 2560, 64, 0)
    assert short < L.verify_attn_paged_workspace_bytes(d, 64 * 32, 64, 0)
    # chunks 8..38 resident plus the block's chunk 39: a packed context of 32 chunks
    assert L.verify_attn_paged_resident(d, P, P, P, P, _i32(*range(8, 40)), 32, 160, 2560, 0,
                                        P, short, P, NULL, NULL) == EWS


def test_device_position_checks():
    """The calls that read the block's position from device memory refuse on the host what the
    position-argument calls refuse, plus a null position, a negative cap and prefill-sized
    blocks; their split layout and workspace are those of the largest position."""
    ws_ring = L.verify_attn_ring_workspace_bytes(dims(), 2048, 512, 0)
    rd = lambda d=None, pos=P, cap=200000, size=2048, window=512, splits=0, ws=P, wsb=ws_ring, out=P: \
        L.verify_attn_ring_dev(dims() if d is None else d, P, P, P, pos, cap, size, window,  # noqa: E731
                               splits, ws, wsb, out, NULL, NULL)
    assert rd(pos=NULL) == ENULL and rd(out=NULL) == ENULL
    assert rd(cap=-1) == EARG and rd(window=0) == EARG and rd(splits=-1) == EARG
    assert rd(size=512) == ERING and rd(size=2000) == ERING
    assert rd(d=dims(dtype=0)) == EDTYPE
    assert rd(d=dims(q_len=65)) == ESHAPE                 # 260 rows per KV head: prefill-sized
    assert rd(ws=NULL) == EWS and rd(wsb=ws_ring - 8192 - 1) == EWS   # partials do not fit
    cap = 131056
    ws_pool = L.verify_attn_paged_workspace_bytes(dims(), cap + 16, 64, 0)
    pd = lambda d=None, pos=P, cap=cap, n_table=2048, chunk=64, ws=P, wsb=ws_pool: \
        L.verify_attn_paged_dev(dims() if d is None else d, P, P, P, P, n_table, 2048, chunk,  # noqa: E731
                                pos, cap, 0, ws, wsb, P, NULL, NULL)
    assert pd(pos=NULL) == ENULL and pd(d=None) != ENULL
    assert L.verify_attn_paged_dev(None, P, P, P, P, 2048, 2048, 64, P, cap, 0, P, ws_pool, P,
                                   NULL, NULL) == ENULL
    assert pd(cap=-1) == EARG
    assert pd(cap=cap + 1) == ETABLE                      # position 131,072 needs entry 2,048
    assert pd(chunk=32) == ETABLE
    assert pd(d=dims(q_len=65), cap=cap - 64) == ESHAPE
    assert pd(ws=NULL) == EWS and pd(wsb=ws_pool - 1) == EWS
    ar = lambda n=16, pos=P, cap=100, size=2048: L.verify_kv_append_ring_dev(  # noqa: E731
        P, P, n, pos, cap, 4, 128, P, P, size, NULL)
    assert ar(pos=NULL) == ENULL and ar(cap=-1) == EARG and ar(n=0) == EARG
    assert ar(n=1025) == EARG and ar(size=100) == ERING
    ap = lambda n=16, pos=P, cap=100, n_table=2, table=P: L.verify_kv_append_paged_dev(  # noqa: E731
        P, P, n, pos, cap, 4, 128, P, P, table, n_table, 8, NULL)
    assert ap(pos=NULL) == ENULL and ap(table=NULL) == ENULL and ap(cap=-1) == EARG
    assert ap(cap=113) == ETABLE                          # 113 + 16 - 1 = 128: chunk 2
    assert L.verify_pos_advance(NULL, P, NULL) == ENULL
    assert L.verify_pos_advance(P, NULL, NULL) == ENULL
    # the append inside the attention launch: both row pointers, 16-byte alignment, then the
    # checks of the attention call itself
    odd = ctypes.c_void_p(0x1008)
    rr = lambda kn=P, vn=P, store=P, pos=P, ws=P: L.verify_attn_ring_append_dev(  # noqa: E731
        dims(), P, kn, vn, store, P, pos, 200000, 2048, 512, 0, ws, ws_ring, P, NULL, NULL)
    assert rr(kn=NULL) == ENULL and rr(vn=NULL) == ENULL and rr(store=NULL) == ENULL
    assert rr(kn=odd) == EARG and rr(store=odd) == EARG
    assert rr(pos=NULL) == ENULL and rr(ws=NULL) == EWS
    pr = lambda kn=P, vn=P, pos=P, cap=cap: L.verify_attn_paged_append_dev(  # noqa: E731
        dims(), P, kn, vn, P, P, P, 2048, 2048, 64, pos, cap, 0, P, ws_pool, P, NULL, NULL)
    assert pr(kn=NULL) == ENULL and pr(vn=odd) == EARG
    assert pr(pos=NULL) == ENULL and pr(cap=cap + 1) == ETABLE
