"""A verify step (ring layers, a paged layer, the accept) captured in a HIP graph and replayed:
every replay must reproduce the eager results bit for bit, with eager work and
synchronisations between the replays; and one accept workspace serves many calls in a row."""
import numpy as np
import pytest
import torch

import ring_kv_amd as rk
from synth import accept_case, paged_case, ring_case
from gpu_util import dev, say

pytestmark = pytest.mark.gpu


def test_accept_workspace_reused_many_times():
    ws = torch.zeros(rk.lib().verify_accept_workspace_bytes(16, 65536), dtype=torch.uint8, device="cuda")
    for i in range(12):
        c = accept_case(30, i, 16, 65536, 1e-3, "binomial")
        a, com, _ = rk.verify_accept(dev(c.logits), dev(c.proposals), workspace=ws)
        torch.cuda.synchronize()
        assert int(a.cpu()[0]) == c.planted_accept, f"call {i}"
        assert list(com.cpu().numpy()[:c.planted_accept]) == list(c.proposals[:c.planted_accept])


def test_graph_replay_matches_eager():
    rings = [ring_case(31, l, 131056, 16, 16, 4, 128, 2048, 512, keep_rows=False) for l in range(2)]
    paged = paged_case(31, 9, 16384, 16, 16, 4, 128, keep_rows=False)
    acc = accept_case(31, 0, 16, 65536, 1e-3, "binomial")
    R = [dict(q=dev(c.q), k=dev(c.k_ring), v=dev(c.v_ring), pos0=c.pos0,
              out=torch.empty(16, 16, 128, device="cuda"), lse=torch.empty(16, 16, device="cuda"))
         for c in rings]
    P = dict(q=dev(paged.q), k=dev(paged.k_pool), v=dev(paged.v_pool), pt=dev(paged.page_table),
             out=torch.empty(16, 16, 128, device="cuda"), lse=torch.empty(16, 16, device="cuda"))
    S = rk.verify_attn_paged_auto_splits(16, 4, 128, 16, 16384)
    import ctypes
    from ring_kv_amd._lib import AttnDims
    dims = AttnDims(16, 16, 4, 128, 0.0, 1)
    wsp = torch.empty(rk.lib().verify_attn_paged_workspace_bytes(ctypes.byref(dims), 16384, 64, 0),
                      dtype=torch.uint8, device="cuda")
    wsa = torch.zeros(rk.lib().verify_accept_workspace_bytes(16, 65536), dtype=torch.uint8, device="cuda")
    lg, pr = dev(acc.logits), dev(acc.proposals)
    a_len = torch.empty(1, dtype=torch.int32, device="cuda")
    com = torch.empty(17, dtype=torch.int32, device="cuda")
    amax = torch.empty(17, dtype=torch.int32, device="cuda")

    def step():
        for d in R:
            rk.verify_attn_ring(d["q"], d["k"], d["v"], d["pos0"], 512, out=d["out"], lse=d["lse"])
        rk.verify_attn_paged(P["q"], P["k"], P["v"], P["pt"], 16384, out=P["out"], lse=P["lse"],
                             workspace=wsp)
        rk.verify_accept(lg, pr, accept_len=a_len, committed=com, row_argmax=amax, workspace=wsa)

    def snapshot():
        torch.cuda.synchronize()
        return [t.clone() for t in (R[0]["out"], R[0]["lse"], R[1]["out"], R[1]["lse"], P["out"],
                                    P["lse"], a_len, com, amax)]

    say("graph: eager reference")
    step()
    ref = snapshot()
    assert int(a_len.cpu()[0]) == acc.planted_accept
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    say("graph: capture")
    with torch.cuda.graph(g):
        step()
    for rep in range(5):
        for t in (R[0]["out"], P["out"], com):
            t.fill_(-7)                       # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        got = snapshot()
        say(f"graph: replay {rep}")
        for a, b in zip(got, ref):
            assert torch.equal(a, b), f"replay {rep} differs from the eager step"
