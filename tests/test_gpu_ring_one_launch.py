"""The ring layer in one launch: the split workgroups of each (KV head, row tile) merge that
tile's partials inside the split launch, using counters at the start of the ring call's
workspace.  Against the two-launch form (a workspace without room for the counters) the bits
must be the same; against the fp64 oracle, the bf16 tolerance; the arrival counters (the first
word of each group's 128-byte line) must be zero after every call, eager or replayed from a
graph."""
import ctypes

import numpy as np
import pytest
import torch

import ring_kv_amd as rk
from ring_kv_amd._lib import AttnDims
from synth import ring_case
from gpu_util import assert_attn_close, dev, run_oracle, say

pytestmark = pytest.mark.gpu

COUNTER_BYTES = 8192


def _arrivals_zero(ws):
    """The arrival counter of every group (word 0 of its 128-byte line) is zero; the line's
    generation word may hold anything."""
    return int(ws[:COUNTER_BYTES].view(torch.int32).view(-1, 32)[:, 0].count_nonzero()) == 0


def _ws_bytes(c):
    hq, hkv = c.q.shape[1], c.k_ring.shape[1]
    dims = AttnDims(c.q_len, hq, hkv, c.q.shape[2], 0.0, 1)
    return rk.lib().verify_attn_ring_workspace_bytes(ctypes.byref(dims), c.ring_size, c.window, 0)


# (pos0, q_len, hq, hkv, d, ring_size, window): the window layers' shape at several positions
# (split counts 2..10), 16-, 32- and 64-row tiles, head_dim 64, a wider window (11 splits); and
# shapes that keep two launches with counters given (row-tile groups not a multiple of 8, more
# than 12 splits)
CASES = [
    (30000, 16, 16, 4, 128, 2048, 512),
    (30720, 16, 16, 4, 128, 2048, 512),
    (2040, 16, 16, 4, 128, 2048, 512),
    (100, 16, 16, 4, 128, 2048, 512),
    (20000, 16, 16, 4, 64, 2048, 512),
    (5000, 16, 16, 4, 128, 640, 600),
    (9000, 16, 8, 2, 128, 2048, 512),
    (9000, 16, 16, 8, 128, 2048, 512),
    (9000, 64, 16, 4, 128, 2048, 512),
    (20000, 17, 16, 4, 128, 2048, 512),
    (20000, 16, 16, 4, 128, 2048, 1000),
]


@pytest.mark.parametrize("pos0,q_len,hq,hkv,d,R,W", CASES)
def test_one_launch_equals_two_launches(pos0, q_len, hq, hkv, d, R, W):
    c = ring_case(971, pos0, pos0, q_len, hq, hkv, d, R, W)
    q, kr, vr = dev(c.q), dev(c.k_ring), dev(c.v_ring)
    full = _ws_bytes(c)
    say(f"ring one launch pos0={pos0} q_len={q_len} hq={hq} hkv={hkv} d={d} R={R} W={W} "
        f"workspace {full}")
    assert full > COUNTER_BYTES
    ws = torch.zeros(full, dtype=torch.uint8, device="cuda")
    o1, l1 = rk.verify_attn_ring(q, kr, vr, pos0, W, workspace=ws)
    o1b, l1b = rk.verify_attn_ring(q, kr, vr, pos0, W, workspace=ws)       # counters reused
    # the two-launch form: a workspace one counter block short, through the C interface (the
    # binding insists on the full size)
    short = torch.empty(full - COUNTER_BYTES, dtype=torch.uint8, device="cuda")
    o2 = torch.empty_like(o1)
    l2 = torch.empty_like(l1)
    dims = AttnDims(q_len, hq, hkv, d, 0.0, 1)
    ptr = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    st = rk.lib().verify_attn_ring(
        ctypes.byref(dims), ptr(q), ptr(kr), ptr(vr), pos0, pos0 % R, R, W, 0, ptr(short),
        short.numel(), ptr(o2), ptr(l2), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, st
    torch.cuda.synchronize()
    assert _arrivals_zero(ws), "counters not left zero"
    assert torch.equal(o1, o2) and torch.equal(l1, l2), "one launch differs from two launches"
    assert torch.equal(o1, o1b) and torch.equal(l1, l1b)
    assert_attn_close((o1.cpu().numpy(), l1.cpu().numpy()), run_oracle(c), "bf16",
                      f"ring one launch pos0={pos0}")


def test_one_launch_graph_replays():
    """The counters reset themselves: a captured call replayed with its outputs clobbered
    between replays gives the eager bits every time and leaves the arrival counters zero."""
    c = ring_case(972, 0, 30000, 16, 16, 4, 128, 2048, 512)
    q, kr, vr = dev(c.q), dev(c.k_ring), dev(c.v_ring)
    ws = torch.zeros(_ws_bytes(c), dtype=torch.uint8, device="cuda")
    out = torch.empty((16, 16, 128), dtype=torch.float32, device="cuda")
    lse = torch.empty((16, 16), dtype=torch.float32, device="cuda")
    say("ring one launch: eager")
    rk.verify_attn_ring(q, kr, vr, 30000, 512, out=out, lse=lse, workspace=ws)
    torch.cuda.synchronize()
    want_o, want_l = out.clone(), lse.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        rk.verify_attn_ring(q, kr, vr, 30000, 512, out=out, lse=lse, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        rk.verify_attn_ring(q, kr, vr, 30000, 512, out=out, lse=lse, workspace=ws)
    for k in range(6):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        say(f"ring one launch: replay {k}")
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, want_o) and torch.equal(lse, want_l), f"replay {k}"
        assert _arrivals_zero(ws), f"replay {k}: counters"
    assert_attn_close((out.cpu().numpy(), lse.cpu().numpy()), run_oracle(c), "bf16",
                      "ring one launch replayed")


def test_counters_not_zeroed_give_nan_not_mixed_rows():
    """Counters the caller did not zero (every byte 0x18 here: more arrivals than the group has)
    cannot pass for a complete group: the layer writes NaN rather than rows merged from partials
    that may not be there.  Zeroed again, the same workspace gives the exact result."""
    c = ring_case(973, 0, 30000, 16, 16, 4, 128, 2048, 512)
    q, kr, vr = dev(c.q), dev(c.k_ring), dev(c.v_ring)
    full = _ws_bytes(c)
    ws = torch.full((full,), 0x18, dtype=torch.uint8, device="cuda")
    say("ring one launch: counters not zeroed")
    o, l = rk.verify_attn_ring(q, kr, vr, 30000, 512, workspace=ws)
    torch.cuda.synchronize()
    assert torch.isnan(o).all() and torch.isnan(l).all()
    ws[:COUNTER_BYTES].zero_()
    o2, l2 = rk.verify_attn_ring(q, kr, vr, 30000, 512, workspace=ws)
    torch.cuda.synchronize()
    assert _arrivals_zero(ws)
    assert_attn_close((o2.cpu().numpy(), l2.cpu().numpy()), run_oracle(c), "bf16",
                      "ring one launch after zeroing")


def test_one_workspace_across_split_counts():
    """One workspace serves calls whose split counts differ (positions whose window spans 2 to 10
    chunks, in an order that goes up and down): each call's arrival counters start from zero
    whatever the previous call's split count was, and each call gives the two-launch bits."""
    dims = AttnDims(16, 16, 4, 128, 0.0, 1)
    full = rk.lib().verify_attn_ring_workspace_bytes(ctypes.byref(dims), 2048, 512, 0)
    ws = torch.zeros(full, dtype=torch.uint8, device="cuda")
    for k, pos0 in enumerate((30000, 100, 30720, 470, 2040, 30016, 60, 30000)):
        c = ring_case(974 + k, pos0, pos0, 16, 16, 4, 128, 2048, 512)
        q, kr, vr = dev(c.q), dev(c.k_ring), dev(c.v_ring)
        say(f"ring one launch, shared workspace: pos0={pos0}")
        o1, l1 = rk.verify_attn_ring(q, kr, vr, pos0, 512, workspace=ws)
        o2, l2 = rk.verify_attn_ring(q, kr, vr, pos0, 512,
                                     workspace=torch.empty(full - COUNTER_BYTES,
                                                           dtype=torch.uint8, device="cuda"))
        torch.cuda.synchronize()
        assert _arrivals_zero(ws), f"pos0={pos0}: counters"
        assert torch.equal(o1, o2) and torch.equal(l1, l2), f"pos0={pos0}: one launch differs"
        assert not torch.isnan(o1).any()
