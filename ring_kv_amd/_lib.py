"""ctypes view of libring_kv (include/ring_kv.h).  Loading fails loudly if the library has
not been built; there is no other implementation to fall back to."""
from __future__ import annotations

import ctypes
import os
import re
from ctypes import POINTER, c_char_p, c_float, c_int32, c_int64, c_size_t, c_void_p

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libring_kv.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "ring_kv.h")

RKV_F32, RKV_BF16 = 0, 1
STATUS = {0: "RKV_OK", -1: "RKV_ERR_NULL", -2: "RKV_ERR_SHAPE", -3: "RKV_ERR_DTYPE",
          -4: "RKV_ERR_RING", -5: "RKV_ERR_TABLE", -6: "RKV_ERR_WORKSPACE", -7: "RKV_ERR_HIP",
          -8: "RKV_ERR_ARG"}


class AttnDims(ctypes.Structure):
    _fields_ = [("q_len", c_int32), ("n_q_heads", c_int32), ("n_kv_heads", c_int32),
                ("head_dim", c_int32), ("scale", c_float), ("dtype", c_int32)]


class RkvError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn}: {STATUS.get(status, status)} ({msg})")
        self.status = status


_P = c_void_p
_DIMS = POINTER(AttnDims)
_PROTOS = {
    "rkv_abi_version": (c_int32, []),
    "rkv_status_str": (c_char_p, [c_int32]),
    "decode_attn_ref_layout_workspace_bytes": (c_size_t, [_DIMS, c_int64, c_int32]),
    "decode_attn_ref_layout": (c_int32, [_DIMS, _P, _P, _P, c_int64, c_int32, c_int32, _P,
                                         c_size_t, _P, _P, _P]),
    "verify_attn_ring_workspace_bytes": (c_size_t, [_DIMS, c_int32, c_int32, c_int32]),
    "verify_attn_ring": (c_int32, [_DIMS, _P, _P, _P, c_int64, c_int32, c_int32, c_int32,
                                   c_int32, _P, c_size_t, _P, _P, _P]),
    "verify_attn_paged_workspace_bytes": (c_size_t, [_DIMS, c_int64, c_int32, c_int32]),
    "verify_attn_paged": (c_int32, [_DIMS, _P, _P, _P, _P, c_int32, c_int32, c_int32, c_int64,
                                    c_int32, _P, c_size_t, _P, _P, _P]),
    "verify_attn_paged_auto_splits": (c_int32, [_DIMS, c_int64, c_int32]),
    "verify_attn_paged_noalloc": (c_int32, [_DIMS, _P, _P, _P, _P, c_int32, c_int32, c_int32,
                                            c_int64, c_int32, _P, _P, _P]),
    "verify_attn_paged_partial": (c_int32, [_DIMS, _P, _P, _P, _P, c_int32, c_int32, c_int32,
                                            c_int64, c_int32, _P, _P, _P]),
    "attn_merge_partials": (c_int32, [_DIMS, c_int32, _P, _P, _P, _P, _P]),
    "verify_accept_workspace_bytes": (c_size_t, [c_int32, c_int32]),
    "verify_accept": (c_int32, [_P, c_int32, c_int32, _P, _P, _P, _P, _P, c_size_t, _P]),
    "ref_layout_to_ring": (c_int32, [_P, _P, c_int64, c_int64, c_int32, c_int32, c_int32, _P,
                                     _P, c_int32, _P]),
    "ref_layout_to_paged": (c_int32, [_P, _P, c_int64, c_int64, c_int32, c_int32, c_int32, _P,
                                      _P, _P, c_int32, c_int32, c_int32, _P]),
    "rkv_pager_create": (c_void_p, [c_int32, c_int32]),
    "rkv_pager_destroy": (None, [c_void_p]),
    "rkv_pager_ctx_len": (c_int64, [c_void_p]),
    "rkv_pager_free_slots": (c_int32, [c_void_p]),
    "rkv_pager_table": (c_int32, [c_void_p, _P, c_int32]),
    "rkv_pager_reserve": (c_int32, [c_void_p, c_int32, _P, _P, _P]),
    "rkv_pager_commit": (c_int32, [c_void_p, c_int32]),
    "verify_kv_append_ring": (c_int32, [_P, _P, c_int32, c_int64, c_int32, c_int32, _P, _P,
                                        c_int32, _P]),
    "verify_kv_append_paged": (c_int32, [_P, _P, c_int32, c_int64, c_int32, c_int32, _P, _P, _P,
                                         c_int32, c_int32, c_int32, c_int32, _P, _P]),
    "kv_page_workspace_bytes": (c_size_t, [c_int32, c_int32, c_int32]),
    "kv_page_out": (c_int32, [_P, _P, c_int32, c_int32, c_int32, _P, _P, c_int32, _P, _P, c_int64,
                              _P, c_size_t, _P]),
    "kv_page_in": (c_int32, [_P, _P, c_int64, _P, _P, c_int32, _P, _P, c_int32, c_int32, c_int32,
                             _P, c_size_t, _P]),
    "verify_attn_paged_resident": (c_int32, [_DIMS, _P, _P, _P, _P, _P, c_int32, c_int32, c_int64,
                                             c_int32, _P, c_size_t, _P, _P, _P]),
    "verify_attn_ring_dev": (c_int32, [_DIMS, _P, _P, _P, _P, c_int64, c_int32, c_int32, c_int32,
                                       _P, c_size_t, _P, _P, _P]),
    "verify_attn_paged_dev": (c_int32, [_DIMS, _P, _P, _P, _P, c_int32, c_int32, c_int32, _P,
                                        c_int64, c_int32, _P, c_size_t, _P, _P, _P]),
    "verify_attn_ring_append_dev": (c_int32, [_DIMS, _P, _P, _P, _P, _P, _P, c_int64, c_int32,
                                              c_int32, c_int32, _P, c_size_t, _P, _P, _P]),
    "verify_attn_paged_append_dev": (c_int32, [_DIMS, _P, _P, _P, _P, _P, _P, c_int32, c_int32,
                                               c_int32, _P, c_int64, c_int32, _P, c_size_t, _P,
                                               _P, _P]),
    "verify_kv_append_ring_dev": (c_int32, [_P, _P, c_int32, _P, c_int64, c_int32, c_int32, _P,
                                            _P, c_int32, _P]),
    "verify_kv_append_paged_dev": (c_int32, [_P, _P, c_int32, _P, c_int64, c_int32, c_int32, _P,
                                             _P, _P, c_int32, c_int32, _P]),
    "verify_pos_advance": (c_int32, [_P, _P, _P]),
    "rkv_pager_evict": (c_int32, [c_void_p, _P, c_int32, _P]),
    "rkv_pager_restore": (c_int32, [c_void_p, _P, c_int32, _P]),
    "rkv_pager_resident": (c_int32, [c_void_p, _P, _P, c_int32]),
}

_lib = None


def declared_functions() -> list[str]:
    """Function names the public header declares."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(
        r"^\s*(?:const\s+)?(?:int32_t|int64_t|size_t|void|rkv_pager|char)\s*\**\s*(\w+)\s*\(",
        text, flags=re.M)))


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m ring_kv_amd.build` "
                               "(libring_kv has no fallback implementation)")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _PROTOS.items():
            f = getattr(l, name)
            f.restype = res
            f.argtypes = args
        _lib = l
    return _lib


def check(fn: str, status: int) -> None:
    if status != 0:
        raise RkvError(fn, status, lib().rkv_status_str(status).decode())
