"""One captured verify step replayed as the decode loop: the block's position lives in device
memory, so a single HIP graph of append -> window / full attention -> greedy accept -> advance
serves every step while the context grows by the a + 1 tokens each step commits.  Each replay is
checked against the oracle's decode sequence (the cache oracle's appends and the attention
oracle over the ring and the pool, and the plain contiguous definition over the committed
history); the stores are compared bit for bit at the end.  Also: the device-position calls
against the position-argument calls, and a position outside the captured range."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import ring_kv_amd as rk
from ring_kv_amd._lib import AttnDims
from synth import accept_case, paged_case, paged_store, ring_case, ring_store, \
    round_f32_to_bf16_bits
from gpu_util import REL_BF16, TOL_BF16, TOL_LSE_BF16, dev, say

pytestmark = pytest.mark.gpu

CH = 64
HQ, HKV, D, Q, W, R = 16, 4, 128, 16, 512, 2048


def _bits(g, shape):
    return round_f32_to_bf16_bits(g.standard_normal(shape).astype(np.float32))


def _host(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _close(got, want, what):
    out, lse = got
    o_ref, l_ref = want
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse)), f"{what}: non-finite output"
    err, lerr = float(np.abs(out - o_ref).max()), float(np.abs(lse - l_ref).max())
    assert err <= TOL_BF16 and err <= REL_BF16 * np.abs(o_ref).max(), f"{what}: error {err}"
    assert lerr <= TOL_LSE_BF16, f"{what}: lse error {lerr}"
    return err, lerr


@pytest.mark.parametrize("fused,P0,N", [(False, 9000, 10), (True, 9000, 10), (True, 131000, 4)],
                         ids=["append_then_attend", "append_in_attention",
                              "append_in_attention_131k"])
def test_one_graph_replayed_over_decode_steps(fused, P0, N):
    """Four layers (three window layers over 2,048-slot rings, one full-attention layer over a
    permuted pool) at a context of 9,000 committed positions, ten decode steps from one graph;
    and at 131,000 (the 40-layer step's context) for four steps.
    Each step: the block's 16 K/V rows are appended at the device position in every layer, each
    layer attends, the accept runs over [16 x 4,096] logits with a planted agreement prefix, and
    the position advances by a + 1 on the device.  The block is the last committed token and 15
    drafts (rows at positions P .. P+15), so the a accepted drafts keep rows P .. P+a, all of them
    written by this step's append, and the next block starts at P + a + 1.  The host copies step
    k's inputs into the captured buffers and replays; nothing else changes between steps.  Run
    with the append and the attention as two calls per layer, and as one (the append inside the
    attention launch)."""
    g = np.random.default_rng(2026)
    kinds = ["ring", "ring", "ring", "paged"]
    V = 4096
    pos_cap = P0 + Q * N
    n_table = -(-(pos_cap + Q) // CH)          # every chunk any step can reach, reserved
    n_slots = n_table + 5
    pt = g.permutation(n_slots)[:n_table].astype(np.int32)
    # committed history of every layer, positions 0 .. P0-1, and room for the steps
    hist = [(_bits(g, (pos_cap + Q, HKV, D)), _bits(g, (pos_cap + Q, HKV, D))) for _ in kinds]
    host, gpu = [], []
    for kind, (hk, hv) in zip(kinds, hist):
        if kind == "ring":
            kr, vr = ring_store(hk[P0 - R:P0], hv[P0 - R:P0], P0 - R, R)
            host.append([kr, vr])
            gpu.append([dev(kr), dev(vr)])
        else:
            kp, vp = paged_store(hk[:P0], hv[:P0], pt, n_slots)      # unwritten slots hold NaN
            host.append([kp, vp])
            gpu.append([dev(kp), dev(vp)])
    d_pt = dev(pt)
    # every step's inputs, resident on the device
    steps = []
    for k in range(N):
        ac = accept_case(60, k, Q - 1, V, 0.0, "uniform")
        steps.append(dict(q=[_bits(g, (Q, HQ, D)) for _ in kinds],
                          kn=[_bits(g, (Q, HKV, D)) for _ in kinds],
                          vn=[_bits(g, (Q, HKV, D)) for _ in kinds], acc=ac))
    dsteps = [dict(q=[dev(x) for x in s["q"]], kn=[dev(x) for x in s["kn"]],
                   vn=[dev(x) for x in s["vn"]], lg=dev(s["acc"].logits),
                   pr=dev(s["acc"].proposals)) for s in steps]
    # the captured buffers
    qb = [torch.empty(Q, HQ, D, dtype=torch.bfloat16, device="cuda") for _ in kinds]
    kb = [torch.empty(Q, HKV, D, dtype=torch.bfloat16, device="cuda") for _ in kinds]
    vb = [torch.empty(Q, HKV, D, dtype=torch.bfloat16, device="cuda") for _ in kinds]
    outs = [torch.empty(Q, HQ, D, device="cuda") for _ in kinds]
    lses = [torch.empty(Q, HQ, device="cuda") for _ in kinds]
    lg = torch.empty(Q, V, device="cuda")
    pr = torch.empty(Q - 1, dtype=torch.int32, device="cuda")
    a_len = torch.empty(1, dtype=torch.int32, device="cuda")
    com = torch.empty(Q, dtype=torch.int32, device="cuda")
    amax = torch.empty(Q, dtype=torch.int32, device="cuda")
    d_pos = torch.tensor([P0], dtype=torch.int64, device="cuda")
    L = rk.lib()
    dims = AttnDims(Q, HQ, HKV, D, 0.0, 1)
    ws_r = torch.zeros(L.verify_attn_ring_workspace_bytes(ctypes.byref(dims), R, W, 0),
                       dtype=torch.uint8, device="cuda")
    ws_p = torch.empty(L.verify_attn_paged_workspace_bytes(ctypes.byref(dims), pos_cap + Q, CH, 0),
                       dtype=torch.uint8, device="cuda")
    ws_a = torch.zeros(L.verify_accept_workspace_bytes(Q - 1, V), dtype=torch.uint8, device="cuda")

    def step():
        for i, kind in enumerate(kinds):
            k_st, v_st = gpu[i]
            if fused and kind == "ring":
                rk.verify_attn_ring_append_dev(qb[i], kb[i], vb[i], k_st, v_st, d_pos, pos_cap, W,
                                               out=outs[i], lse=lses[i], workspace=ws_r)
            elif fused:
                rk.verify_attn_paged_append_dev(qb[i], kb[i], vb[i], k_st, v_st, d_pt, d_pos,
                                                pos_cap, out=outs[i], lse=lses[i], workspace=ws_p)
            elif kind == "ring":
                rk.verify_kv_append_ring_dev(kb[i], vb[i], d_pos, pos_cap, k_st, v_st)
                rk.verify_attn_ring_dev(qb[i], k_st, v_st, d_pos, pos_cap, W, out=outs[i],
                                        lse=lses[i], workspace=ws_r)
            else:
                rk.verify_kv_append_paged_dev(kb[i], vb[i], d_pos, pos_cap, k_st, v_st, d_pt)
                rk.verify_attn_paged_dev(qb[i], k_st, v_st, d_pt, d_pos, pos_cap, out=outs[i],
                                         lse=lses[i], workspace=ws_p)
        rk.verify_accept(lg, pr, accept_len=a_len, committed=com, row_argmax=amax, workspace=ws_a)
        rk.verify_pos_advance(d_pos, a_len)

    graph = torch.cuda.CUDAGraph()
    say("decode loop: capture")
    with torch.cuda.graph(graph):
        step()
    P = P0
    for k in range(N):
        s, ds = steps[k], dsteps[k]
        for i in range(len(kinds)):
            qb[i].copy_(ds["q"][i])
            kb[i].copy_(ds["kn"][i])
            vb[i].copy_(ds["vn"][i])
            outs[i].fill_(float("nan"))
            lses[i].fill_(float("nan"))
        lg.copy_(ds["lg"])
        pr.copy_(ds["pr"])
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        # the oracle's step: append, attend, accept, advance
        errs = []
        for i, kind in enumerate(kinds):
            hk, hv = hist[i]
            hk[P:P + Q], hv[P:P + Q] = s["kn"][i], s["vn"][i]
            got = (outs[i].cpu().numpy(), lses[i].cpu().numpy())
            if kind == "ring":
                host[i] = list(oracle.append_ring(*host[i], s["kn"][i], s["vn"][i], P))
                want = oracle.attention_ring(s["q"][i], *host[i], P, P % R, R, W)
                # the same window over the history from the first key any query sees (the
                # positions shift together, the window's keys stay the same)
                lo = max(0, P - W + 1)
                plain = oracle.attention_contiguous(s["q"][i], hk[lo:], hv[lo:], P + Q - lo,
                                                    window=W, dtype="bf16")
            else:
                host[i] = list(oracle.append_paged(*host[i], pt, s["kn"][i], s["vn"][i], P))
                want = oracle.attention_paged(s["q"][i], *host[i], pt, P + Q)
                plain = oracle.attention_contiguous(s["q"][i], hk, hv, P + Q, dtype="bf16")
            np.testing.assert_allclose(want[0], plain[0], rtol=0, atol=1e-12)
            errs.append(_close(got, want, f"step {k} layer {i} ({kind}) at position {P}")[0])
        ra, rcom, rt = oracle.greedy_accept(s["acc"].logits, s["acc"].proposals)
        assert ra == s["acc"].planted_accept
        a = int(a_len.cpu()[0])
        assert a == ra, f"step {k}: accept length {a}, oracle {ra}"
        assert list(com.cpu().numpy()) == list(rcom) + [-1] * (Q - 1 - ra)
        assert list(amax.cpu().numpy()) == list(rt)
        P += ra + 1
        assert int(d_pos.cpu()[0]) == P, f"step {k}: device position {int(d_pos.cpu()[0])}, want {P}"
        say(f"decode loop step {k}: accept {a}, next position {P}, max|err| {max(errs):.2e}")
    for i in range(len(kinds)):
        np.testing.assert_array_equal(_host(gpu[i][0]), host[i][0])
        np.testing.assert_array_equal(_host(gpu[i][1]), host[i][1])


@pytest.mark.parametrize("pos0", [100, 2040, 30000, 30720])
def test_ring_dev_equals_ring_call(pos0):
    """The device-position ring call gives the position-argument call's bits: the same chunk
    per split, the widest span's extra split empty (it weighs exactly 0 in the merge)."""
    c = ring_case(61, 0, pos0, Q, HQ, HKV, D, R, W, keep_rows=False)
    q, kr, vr = dev(c.q), dev(c.k_ring), dev(c.v_ring)
    say(f"ring dev pos0={pos0}")
    o1, l1 = rk.verify_attn_ring(q, kr, vr, pos0, W)
    d_pos = torch.tensor([pos0], dtype=torch.int64, device="cuda")
    o2, l2 = rk.verify_attn_ring_dev(q, kr, vr, d_pos, pos0 + 1000, W)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("ctx", [8192, 8207, 65])
def test_paged_dev_equals_paged_call(ctx):
    """At pos_cap = the position itself the split layout is the position call's: same bits.  A
    larger cap splits as for its own context: the oracle's result within tolerance."""
    n = -(-ctx // CH)
    c = paged_case(62, 0, ctx, Q, HQ, HKV, D, n_slots=n + 40, keep_rows=False)
    # table entries past the context: the slots the context does not use (never read here)
    pt = np.concatenate([c.page_table, np.setdiff1d(np.arange(n + 40), c.page_table)])
    pt = pt.astype(np.int32)
    q, kp, vp, d_pt = dev(c.q), dev(c.k_pool), dev(c.v_pool), dev(pt)
    say(f"paged dev ctx={ctx}")
    o1, l1 = rk.verify_attn_paged(q, kp, vp, d_pt, ctx)
    d_pos = torch.tensor([ctx - Q], dtype=torch.int64, device="cuda")
    o2, l2 = rk.verify_attn_paged_dev(q, kp, vp, d_pt, d_pos, ctx - Q)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    o3, l3 = rk.verify_attn_paged_dev(q, kp, vp, d_pt, d_pos, ctx - Q + 40 * CH)
    torch.cuda.synchronize()
    want = oracle.attention_paged(c.q, c.k_pool, c.v_pool, c.page_table, ctx)
    _close((o3.cpu().numpy(), l3.cpu().numpy()), want, f"paged dev ctx={ctx}, wider cap")


def test_device_position_outside_the_cap():
    """A device position above pos_cap (or negative): attention writes NaN everywhere, the
    appends write nothing.  Every access stays in bounds (the kernels work at position 0)."""
    c = ring_case(63, 0, 30000, Q, HQ, HKV, D, R, W, keep_rows=False)
    q, kr, vr = dev(c.q), dev(c.k_ring), dev(c.v_ring)
    p = paged_case(64, 0, 4096, Q, HQ, HKV, D, keep_rows=False)
    qp, kp, vp, pt = dev(p.q), dev(p.k_pool), dev(p.v_pool), dev(p.page_table)
    rows = torch.ones(Q, HKV, D, dtype=torch.bfloat16, device="cuda")
    kr0, kp0 = kr.clone(), kp.clone()
    for bad in (30001, -5):
        d_pos = torch.tensor([bad], dtype=torch.int64, device="cuda")
        say(f"out-of-range device position {bad}")
        o, l = rk.verify_attn_ring_dev(q, kr, vr, d_pos, 30000, W)
        assert torch.isnan(o).all() and torch.isnan(l).all()
        d_pos.fill_(4080 if bad > 0 else bad)
        o, l = rk.verify_attn_paged_dev(qp, kp, vp, pt, d_pos, 4080 - 1)
        assert torch.isnan(o).all() and torch.isnan(l).all()
        rk.verify_kv_append_ring_dev(rows, rows, d_pos, 100, kr, vr)
        rk.verify_kv_append_paged_dev(rows, rows, d_pos, 100, kp, vp, pt)
        torch.cuda.synchronize()
        assert torch.equal(kr, kr0) and torch.equal(kp, kp0)


def test_launch_status_ignores_an_earlier_error():
    """An error some earlier HIP call left in the thread's last-error state is not reported by
    a good call of the library: its status is the launch's own.  (Whether the error is still
    there afterwards is the HIP runtime's business: the library neither reads nor clears it.)
    Every buffer is allocated before the error is planted, so that no torch work runs between
    the error and the call (torch checks the last error after its own launches)."""
    # the HIP runtime this process already runs (the one torch loaded and the library uses)
    path = next(ln.split()[-1] for ln in open("/proc/self/maps") if "libamdhip64" in ln)
    hip = ctypes.CDLL(path)
    hip.hipGetLastError.restype = ctypes.c_int
    hip.hipSetDevice.argtypes = [ctypes.c_int]
    c = ring_case(65, 0, 30000, Q, HQ, HKV, D, R, W, keep_rows=False)
    q, kr, vr = dev(c.q), dev(c.k_ring), dev(c.v_ring)
    dims = AttnDims(Q, HQ, HKV, D, 0.0, 1)
    ws = torch.zeros(rk.lib().verify_attn_ring_workspace_bytes(ctypes.byref(dims), R, W, 0),
                     dtype=torch.uint8, device="cuda")
    out = torch.empty(Q, HQ, D, device="cuda")
    lse = torch.empty(Q, HQ, device="cuda")
    torch.cuda.synchronize()
    hip.hipGetLastError()                              # start from a clean state
    assert hip.hipSetDevice(9999) != 0                 # an invalid device: an error, nothing else
    rk.verify_attn_ring(q, kr, vr, 30000, W, out=out, lse=lse, workspace=ws)   # raises unless OK
    left = hip.hipGetLastError()                       # consumed here, before any torch work
    say(f"last error after the library call: {left}")
    torch.cuda.synchronize()
    want = oracle.attention_ring(c.q, c.k_ring, c.v_ring, 30000, 30000 % R, R, W)
    _close((out.cpu().numpy(), lse.cpu().numpy()), want, "ring after an earlier error")


@pytest.mark.parametrize("P", [130040, 130048, 9000, 40])
def test_ring_append_in_attention_equals_two_calls(P):
    """The block's rows appended by the attention launch: the same outputs and the same ring as
    verify_kv_append_ring_dev followed by verify_attn_ring_dev (blocks inside one chunk and
    across a chunk boundary, near the ring's start), and the oracle's append + attention."""
    g = np.random.default_rng(P)
    kn, vn = _bits(g, (Q, HKV, D)), _bits(g, (Q, HKV, D))
    c = ring_case(63, 0, P, Q, HQ, HKV, D, R, W, keep_rows=False)
    q, dkn, dvn = dev(c.q), dev(kn), dev(vn)
    k1, v1 = dev(c.k_ring), dev(c.v_ring)
    k2, v2 = k1.clone(), v1.clone()
    cap = P + 3 * Q
    d_pos = torch.tensor([P], dtype=torch.int64, device="cuda")
    dims = AttnDims(Q, HQ, HKV, D, 0.0, 1)
    full = rk.lib().verify_attn_ring_workspace_bytes(ctypes.byref(dims), R, W, 0)
    ws1 = torch.zeros(full, dtype=torch.uint8, device="cuda")
    ws2 = torch.zeros(full, dtype=torch.uint8, device="cuda")
    say(f"ring append in attention P={P}")
    rk.verify_kv_append_ring_dev(dkn, dvn, d_pos, cap, k1, v1)
    o1, l1 = rk.verify_attn_ring_dev(q, k1, v1, d_pos, cap, W, workspace=ws1)
    o2, l2 = rk.verify_attn_ring_append_dev(q, dkn, dvn, k2, v2, d_pos, cap, W, workspace=ws2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2), "outputs differ from the two calls"
    # bit patterns: slots that hold no position are NaN
    assert torch.equal(k1.view(torch.int16), k2.view(torch.int16)), "ring K differs"
    assert torch.equal(v1.view(torch.int16), v2.view(torch.int16)), "ring V differs"
    kr, vr = oracle.append_ring(c.k_ring, c.v_ring, kn, vn, P)
    np.testing.assert_array_equal(_host(k2), kr)
    np.testing.assert_array_equal(_host(v2), vr)
    _close((o2.cpu().numpy(), l2.cpu().numpy()),
           oracle.attention_ring(c.q, kr, vr, P, P % R, R, W), f"ring append in attention P={P}")


@pytest.mark.parametrize("P", [8184, 8192, 100, 40])
def test_paged_append_in_attention_equals_two_calls(P):
    """As above over a permuted pool whose table already holds the block's chunks."""
    g = np.random.default_rng(P + 1)
    kn, vn = _bits(g, (Q, HKV, D)), _bits(g, (Q, HKV, D))
    cap = P + 3 * Q
    ctx = P + Q
    n = -(-(cap + Q) // CH)                    # chunks any position up to the cap can reach
    c = paged_case(64, 0, ctx, Q, HQ, HKV, D, n_slots=n + 7, keep_rows=False)
    pt = np.concatenate([c.page_table, np.setdiff1d(np.arange(n + 7), c.page_table)])[:n]
    pt = pt.astype(np.int32)
    q, dkn, dvn, d_pt = dev(c.q), dev(kn), dev(vn), dev(pt)
    k1, v1 = dev(c.k_pool), dev(c.v_pool)
    k2, v2 = k1.clone(), v1.clone()
    d_pos = torch.tensor([P], dtype=torch.int64, device="cuda")
    say(f"paged append in attention P={P}")
    rk.verify_kv_append_paged_dev(dkn, dvn, d_pos, cap, k1, v1, d_pt)
    o1, l1 = rk.verify_attn_paged_dev(q, k1, v1, d_pt, d_pos, cap)
    o2, l2 = rk.verify_attn_paged_append_dev(q, dkn, dvn, k2, v2, d_pt, d_pos, cap)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2), "outputs differ from the two calls"
    assert torch.equal(k1.view(torch.int16), k2.view(torch.int16)), "pool K differs"
    assert torch.equal(v1.view(torch.int16), v2.view(torch.int16)), "pool V differs"
    kp, vp = oracle.append_paged(c.k_pool, c.v_pool, pt, kn, vn, P)
    np.testing.assert_array_equal(_host(k2), kp)
    np.testing.assert_array_equal(_host(v2), vp)
    _close((o2.cpu().numpy(), l2.cpu().numpy()), oracle.attention_paged(c.q, kp, vp, pt, ctx),
           f"paged append in attention P={P}")


def test_append_in_attention_outside_the_cap_writes_nothing():
    """A device position above the cap: no row is written and the attention is NaN."""
    g = np.random.default_rng(77)
    kn, vn = _bits(g, (Q, HKV, D)), _bits(g, (Q, HKV, D))
    c = ring_case(65, 0, 30000, Q, HQ, HKV, D, R, W, keep_rows=False)
    q, dkn, dvn = dev(c.q), dev(kn), dev(vn)
    kr, vr = dev(c.k_ring), dev(c.v_ring)
    k0, v0 = kr.clone(), vr.clone()
    d_pos = torch.tensor([30100], dtype=torch.int64, device="cuda")
    say("ring append in attention outside the cap")
    o, l = rk.verify_attn_ring_append_dev(q, dkn, dvn, kr, vr, d_pos, 30000, W)
    torch.cuda.synchronize()
    assert torch.equal(kr.view(torch.int16), k0.view(torch.int16))
    assert torch.equal(vr.view(torch.int16), v0.view(torch.int16))
    assert torch.isnan(o).all() and torch.isnan(l).all()
