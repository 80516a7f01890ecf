"""Helpers for the GPU parity tests: run a synthetic case through the HIP library (via the
C interface) and through the fp64 oracle, and compare."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import ring_kv_amd as rk

# Tolerances: max-abs error of the f32 output against the fp64 oracle, for bf16 K/V with f32
# accumulation and for f32 inputs; the lse (natural log) gets its own bound.
TOL_BF16 = 1e-2
TOL_F32 = 1e-4
TOL_LSE_BF16 = 2e-3
TOL_LSE_F32 = 1e-4
# guard for long contexts where |O| is small: error relative to the largest |O|
REL_BF16 = 2e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(a, device="cuda"):
    return rk.tensor_from_numpy(a, device)


def run_gpu(c, num_splits=0, **kw):
    """The GPU result for an AttnCase through the matching entry point: numpy (out, lse)."""
    q = dev(c.q)
    if c.kind == "paged":
        out, lse = rk.verify_attn_paged(q, dev(c.k_pool), dev(c.v_pool), dev(c.page_table),
                                        c.ctx_len, num_splits=num_splits, **kw)
    elif c.kind == "ring":
        out, lse = rk.verify_attn_ring(q, dev(c.k_ring), dev(c.v_ring), c.pos0, c.window,
                                       num_splits=num_splits, **kw)
    else:
        out, lse = rk.decode_attn_ref_layout(q, dev(c.k_rows), dev(c.v_rows), c.ctx_len, c.window,
                                             num_splits=num_splits, **kw)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def run_oracle(c):
    if c.kind == "paged":
        return oracle.attention_paged(c.q, c.k_pool, c.v_pool, c.page_table, c.ctx_len,
                                      dtype=c.dtype, window=c.window)
    if c.kind == "ring":
        return oracle.attention_ring(c.q, c.k_ring, c.v_ring, c.pos0, c.ring_head, c.ring_size,
                                     c.window, dtype=c.dtype)
    return oracle.attention_contiguous(c.q, c.k_rows, c.v_rows, c.ctx_len, window=c.window,
                                       dtype=c.dtype)


def assert_attn_close(got, want, dtype, what=""):
    out, lse = got
    o_ref, l_ref = want
    assert out.shape == o_ref.shape and lse.shape == l_ref.shape
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse)), f"{what}: non-finite output"
    err = np.abs(out - o_ref).max()
    lerr = np.abs(lse - l_ref).max()
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    ltol = TOL_LSE_BF16 if dtype == "bf16" else TOL_LSE_F32
    scale = np.abs(o_ref).max()
    say(f"{what}: max|err| {err:.3e} (tol {tol:g}), rel {err / scale:.3e}, lse err {lerr:.3e}")
    assert err <= tol, f"{what}: max abs error {err} > {tol}"
    assert lerr <= ltol, f"{what}: lse error {lerr} > {ltol}"
    if dtype == "bf16":
        assert err <= REL_BF16 * scale, f"{what}: error {err} is {err / scale:.3g} of max|O|"
