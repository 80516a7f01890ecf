"""Entry points captured in HIP graphs and replayed (a verify step; prefill blocks, the resident
call and host paging):
every replay must reproduce the eager results bit for bit, with eager work and
synchronisations between the replays; and one accept workspace serves many calls in a row.
The whole 40-layer step at context 131,072 plus its accept, captured in one graph, is checked
replay by replay against the fp64 oracle."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import ring_kv_amd as rk
from ring_kv_amd._lib import AttnDims
from synth import STACK_LAYERS, accept_case, paged_case, ring_case, workload
from gpu_util import REL_BF16, TOL_BF16, TOL_LSE_BF16, dev, run_oracle, say

pytestmark = pytest.mark.gpu


def test_graph_replay_stack_40l_131k_against_oracle():
    """The 40-layer step (30 window layers over the 2,048-slot ring at position 131,056, 10
    full-attention layers over permuted pools at context 131,072) and the greedy accept over
    [17 x 65,536] logits, captured in ONE HIP graph and replayed three times, every output
    clobbered by eager work between replays.  After each replay every layer's out and lse are
    compared with the fp64 oracle (bf16 tolerances) and the accept length and committed tokens
    exactly."""
    L = rk.lib()
    dims = AttnDims(16, 16, 4, 128, 0.0, 1)
    ws_p = torch.empty(L.verify_attn_paged_workspace_bytes(ctypes.byref(dims), 131072, 64, 0),
                       dtype=torch.uint8, device="cuda")
    ws_r = torch.zeros(L.verify_attn_ring_workspace_bytes(ctypes.byref(dims), 2048, 512, 0),
                       dtype=torch.uint8, device="cuda")
    layers, refs = [], []
    acc = None
    for l in range(STACK_LAYERS):
        c, acc = workload("stack_40l_131k", l, keep_rows=False)
        d = dict(kind=c.kind, q=dev(c.q), out=torch.empty(16, 16, 128, device="cuda"),
                 lse=torch.empty(16, 16, device="cuda"))
        if c.kind == "ring":
            d.update(k=dev(c.k_ring), v=dev(c.v_ring), pos0=c.pos0, window=c.window)
        else:
            d.update(k=dev(c.k_pool), v=dev(c.v_pool), pt=dev(c.page_table), ctx=c.ctx_len)
        refs.append(run_oracle(c))
        layers.append(d)
        if l % 8 == 7:
            say(f"stack graph: layer {l} built, oracle done")
        del c
    lg, pr = dev(acc.logits), dev(acc.proposals)
    ra, rcom, rt = oracle.greedy_accept(acc.logits, acc.proposals)
    assert ra == acc.planted_accept
    wsa = torch.zeros(L.verify_accept_workspace_bytes(16, 65536), dtype=torch.uint8, device="cuda")
    a_len = torch.empty(1, dtype=torch.int32, device="cuda")
    com = torch.empty(17, dtype=torch.int32, device="cuda")
    amax = torch.empty(17, dtype=torch.int32, device="cuda")

    def step():
        for d in layers:
            if d["kind"] == "ring":
                rk.verify_attn_ring(d["q"], d["k"], d["v"], d["pos0"], d["window"], out=d["out"],
                                    lse=d["lse"], workspace=ws_r)
            else:
                rk.verify_attn_paged(d["q"], d["k"], d["v"], d["pt"], d["ctx"], out=d["out"],
                                     lse=d["lse"], workspace=ws_p)
        rk.verify_accept(lg, pr, accept_len=a_len, committed=com, row_argmax=amax, workspace=wsa)

    g = torch.cuda.CUDAGraph()
    say("stack graph: capture")
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        for d in layers:
            d["out"].fill_(float("nan"))                 # eager work between replays
            d["lse"].fill_(float("nan"))
        a_len.fill_(-1)
        com.fill_(-7)
        amax.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        worst = (0.0, 0.0)
        for l, (d, (o_ref, l_ref)) in enumerate(zip(layers, refs)):
            out, lse = d["out"].cpu().numpy(), d["lse"].cpu().numpy()
            assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse)), f"replay {rep} layer {l}"
            err, lerr = float(np.abs(out - o_ref).max()), float(np.abs(lse - l_ref).max())
            assert err <= TOL_BF16 and err <= REL_BF16 * np.abs(o_ref).max(), \
                f"replay {rep} layer {l} ({d['kind']}): max abs error {err}"
            assert lerr <= TOL_LSE_BF16, f"replay {rep} layer {l}: lse error {lerr}"
            worst = (max(worst[0], err), max(worst[1], lerr))
        a = int(a_len.cpu()[0])
        assert a == ra, f"replay {rep}: accept length {a}, oracle {ra}"
        assert list(com.cpu().numpy()) == list(rcom) + [-1] * (16 - ra)
        assert list(amax.cpu().numpy()) == list(rt)
        say(f"stack graph: replay {rep}: max|err| out {worst[0]:.2e}, lse {worst[1]:.2e}, "
            f"accept {a} exact")


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


def test_graph_replay_prefill_resident_and_paging():
    """The other entry points in a HIP graph: a 1,024-token prefill block over the pool (matrix-
    core kernel, 4 splits, row-parallel merge) and over the ring (64-row tiles), attention over a
    resident subset, and a page-out to pinned host memory followed by a page-in of long runs
    (copy engines) and of scattered ids (direct kernel).  Every replay reproduces the eager
    results bit for bit, with the outputs, the host store and the target pool clobbered by eager
    work between replays."""
    import ctypes
    from ring_kv_amd._lib import AttnDims
    L = rk.lib()
    pf = paged_case(32, 0, 9216, 1024, 16, 4, 128, keep_rows=False)
    rf = ring_case(33, 0, 30000, 1024, 16, 4, 128, 2048, 512, keep_rows=False)
    vr = paged_case(34, 0, 4096, 16, 16, 4, 128, keep_rows=False)
    Pq, Pk, Pv, Pt = dev(pf.q), dev(pf.k_pool), dev(pf.v_pool), dev(pf.page_table)
    Rq, Rk, Rv = dev(rf.q), dev(rf.k_ring), dev(rf.v_ring)
    Vq, Vk, Vv = dev(vr.q), dev(vr.k_pool), dev(vr.v_pool)
    keep = [0, 3, 5, 9, 10, 11, 20, 31, 40] + list(range(60, 64))
    vslots = dev(np.array([int(vr.page_table[c]) for c in keep], np.int32))
    d16, d1024 = AttnDims(16, 16, 4, 128, 0.0, 1), AttnDims(1024, 16, 4, 128, 0.0, 1)
    ws_pf = torch.empty(L.verify_attn_paged_workspace_bytes(ctypes.byref(d1024), 9216, 64, 0),
                        dtype=torch.uint8, device="cuda")
    ws_res = torch.empty(max(1, L.verify_attn_paged_workspace_bytes(
        ctypes.byref(d16), 64 * len(keep), 64, 0)), dtype=torch.uint8, device="cuda")
    outs = [torch.empty(q, 16, 128, device="cuda") for q in (1024, 1024, 16)]
    lses = [torch.empty(q, 16, device="cuda") for q in (1024, 1024, 16)]
    # paging: 40 pool slots out to 96 host entries, then back into another pool
    hkv, d = 4, 128
    src_k = Vk[:40].clone()
    src_v = Vv[:40].clone()
    kh = torch.zeros((96, hkv, 64, d), dtype=torch.bfloat16, pin_memory=True)
    vh = torch.zeros((96, hkv, d, 64), dtype=torch.bfloat16, pin_memory=True)
    out_slots = list(range(40))
    out_ids = list(range(10, 30)) + [int(x) for x in np.random.default_rng(35).choice(
        np.arange(40, 96), 20, replace=False)]
    dst_k = torch.zeros_like(src_k)
    dst_v = torch.zeros_like(src_v)
    run_ids, run_slots = list(range(10, 30)), list(range(20))            # one long run
    sc_ids, sc_slots = out_ids[20:], list(range(20, 40))                  # scattered
    ws_pg = torch.empty(L.kv_page_workspace_bytes(hkv, d, 40), dtype=torch.uint8, device="cuda")

    def work():
        rk.verify_attn_paged(Pq, Pk, Pv, Pt, 9216, out=outs[0], lse=lses[0], workspace=ws_pf)
        rk.verify_attn_ring(Rq, Rk, Rv, rf.pos0, 512, out=outs[1], lse=lses[1])
        rk.verify_attn_paged_resident(Vq, Vk, Vv, vslots, keep, 4096, out=outs[2], lse=lses[2],
                                      workspace=ws_res)
        rk.kv_page_out(src_k, src_v, out_slots, out_ids, kh, vh, workspace=ws_pg)
        rk.kv_page_in(kh, vh, run_ids, run_slots, dst_k, dst_v, workspace=ws_pg)
        rk.kv_page_in(kh, vh, sc_ids, sc_slots, dst_k, dst_v, workspace=ws_pg)

    def snapshot():
        torch.cuda.synchronize()
        return [t.clone() for t in (*outs, *lses, dst_k, dst_v)] + [kh.clone(), vh.clone()]

    say("graph 2: eager reference")
    work()
    ref = snapshot()
    assert torch.equal(ref[6], src_k) and torch.equal(ref[7], src_v)     # the round trip itself
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        work()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    say("graph 2: capture")
    with torch.cuda.graph(g):
        work()
    for rep in range(4):
        for t in (*outs, *lses):
            t.fill_(-7)                                  # eager work between replays
        dst_k.zero_()
        dst_v.zero_()
        torch.cuda.synchronize()
        kh.zero_()
        vh.zero_()
        g.replay()
        got = snapshot()
        say(f"graph 2: replay {rep}")
        for i, (a, b) in enumerate(zip(got, ref)):
            assert torch.equal(a, b), f"replay {rep}: tensor {i} differs from the eager run"
