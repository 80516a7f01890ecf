"""verify_attn_paged_noalloc (the allocation-free form of verify_attn_paged, its split partials in
the library's static device array) through the C interface: its outputs equal verify_attn_paged's
bit for bit on two calls in a row, the second over a smaller context (fewer splits: the array
keeps the first call's partials past the second's, which must not leak into it); and a call whose
partials exceed the array is refused."""
import ctypes

import numpy as np
import pytest
import torch

import ring_kv_amd as rk
from ring_kv_amd._lib import AttnDims
from synth import paged_case, workload
from gpu_util import dev, say

pytestmark = pytest.mark.gpu

RKV_ERR_WORKSPACE = -6


def _noalloc(c, out, lse):
    L = rk.lib()
    q, kp, vp, pt = dev(c.q), dev(c.k_pool), dev(c.v_pool), dev(c.page_table)
    dims = AttnDims(c.q_len, c.n_q_heads, c.n_kv_heads, c.head_dim, 0.0, 1)
    st = L.verify_attn_paged_noalloc(
        ctypes.byref(dims), ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(kp.data_ptr()),
        ctypes.c_void_p(vp.data_ptr()), ctypes.c_void_p(pt.data_ptr()), pt.numel(),
        kp.shape[0], 64, c.ctx_len, 0, ctypes.c_void_p(out.data_ptr()),
        ctypes.c_void_p(lse.data_ptr()), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    ref_out, ref_lse = rk.verify_attn_paged(q, kp, vp, pt, c.ctx_len)
    torch.cuda.synchronize()
    return st, ref_out, ref_lse


def test_noalloc_equals_workspace_call_twice_in_a_row():
    first, _ = workload("stack_40l_131k", 3, keep_rows=False)      # 64 splits at 131,072
    second = paged_case(70, 0, 8207, 16, 16, 4, 128, keep_rows=False)   # 33 splits
    out = torch.empty(16, 16, 128, device="cuda")
    lse = torch.empty(16, 16, device="cuda")
    for name, c in (("131,072", first), ("8,207", second)):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        say(f"noalloc call at context {name}: "
            f"{rk.verify_attn_paged_auto_splits(16, 4, 128, 16, c.ctx_len)} splits")
        st, ref_out, ref_lse = _noalloc(c, out, lse)
        assert st == 0, f"status {st}"
        assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse), f"context {name}"
        assert bool(torch.isfinite(out).all())


def test_noalloc_refuses_partials_beyond_its_array():
    c = paged_case(71, 0, 9216, 1024, 16, 4, 128, keep_rows=False)     # 1,024-token block: 32 MiB
    L = rk.lib()
    dims = AttnDims(1024, 16, 4, 128, 0.0, 1)
    need = L.verify_attn_paged_workspace_bytes(ctypes.byref(dims), 9216, 64, 0)
    assert need > 16 << 20
    p = ctypes.c_void_p(0x1000)         # refused on the host: never dereferenced
    st = L.verify_attn_paged_noalloc(ctypes.byref(dims), p, p, p, p, c.page_table.size, 144, 64,
                                     9216, 0, p, None, None)
    assert st == RKV_ERR_WORKSPACE
    # one split needs no partials at all
    out = torch.empty(1024, 16, 128, device="cuda")
    q, kp, vp, pt = dev(c.q), dev(c.k_pool), dev(c.v_pool), dev(c.page_table)
    st = L.verify_attn_paged_noalloc(
        ctypes.byref(dims), ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(kp.data_ptr()),
        ctypes.c_void_p(vp.data_ptr()), ctypes.c_void_p(pt.data_ptr()), pt.numel(), kp.shape[0],
        64, 9216, 1, ctypes.c_void_p(out.data_ptr()), None,
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    ref, _ = rk.verify_attn_paged(q, kp, vp, pt, 9216, num_splits=1)
    torch.cuda.synchronize()
    assert st == 0 and torch.equal(out, ref)
    say("noalloc: refusal and the one-split call ok")
