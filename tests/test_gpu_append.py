"""GPU parity of the verify block's KV append (HIP kernels through the C interface) against the
cache oracle: stores and page table bit-exact; and a decode sequence in which every block is
appended, attended and committed, its attention checked against the fp64 oracle on the true
history."""
import numpy as np
import pytest
import torch

import oracle
import ring_kv_amd as rk
from gpu_util import TOL_BF16, TOL_LSE_BF16, dev, say
from synth import round_f32_to_bf16_bits

pytestmark = pytest.mark.gpu
CH = 64


def _bits(g, shape):
    return round_f32_to_bf16_bits(g.standard_normal(shape).astype(np.float32))


def _host(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("pos,n", [(100, 16), (2040, 16), (4090, 16), (0, 1), (131056, 1024),
                                   (5, 2048)])
def test_ring_append_bit_exact(pos, n):
    g = np.random.default_rng(pos + n)
    R, hkv, d = 2048, 4, 128
    kr, vr = _bits(g, (R // CH, hkv, CH, d)), _bits(g, (R // CH, hkv, d, CH))
    kb, vb = _bits(g, (n, hkv, d)), _bits(g, (n, hkv, d))
    say(f"ring append pos={pos} n={n}")
    kd, vd = dev(kr), dev(vr)
    if n > 1024:
        with pytest.raises(rk.RkvError):
            rk.verify_kv_append_ring(dev(kb), dev(vb), pos, kd, vd)
        return
    rk.verify_kv_append_ring(dev(kb), dev(vb), pos, kd, vd)
    wk, wv = oracle.append_ring(kr, vr, kb, vb, pos)
    np.testing.assert_array_equal(_host(kd), wk)
    np.testing.assert_array_equal(_host(vd), wv)


def test_paged_append_bit_exact_with_the_pager():
    g = np.random.default_rng(5)
    n_slots, n_table, hkv, d = 96, 120, 4, 128
    kp, vp = _bits(g, (n_slots, hkv, CH, d)), _bits(g, (n_slots, hkv, d, CH))
    pager, model = rk.Pager(n_slots, n_table), oracle.PagerModel(n_slots, n_table)
    table_dev = torch.full((n_table,), -1, dtype=torch.int32, device="cuda")
    kd, vd = dev(kp), dev(vp)
    for step, (n, keep) in enumerate([(1000, 1000), (1024, 1024), (16, 16), (16, 3), (16, 0),
                                      (64, 64), (16, 16), (1, 1), (700, 650), (16, 9)]):
        kb, vb = _bits(g, (n, hkv, d)), _bits(g, (n, hkv, d))
        ctx = pager.ctx_len
        first, slots = pager.reserve(n)
        assert (first, slots) == model.reserve(n)
        say(f"paged append step {step}: ctx={ctx} n={n} new chunks {slots}")
        rk.verify_kv_append_paged(dev(kb), dev(vb), ctx, kd, vd, table_dev, first, slots)
        kp, vp = oracle.append_paged(kp, vp, model.table, kb, vb, ctx)
        np.testing.assert_array_equal(_host(kd), kp)
        np.testing.assert_array_equal(_host(vd), vp)
        nc = -(-(ctx + n) // CH)
        np.testing.assert_array_equal(table_dev.cpu().numpy()[:nc], np.array(model.table[:nc]))
        pager.commit(keep)
        model.commit(keep)


def test_decode_sequence_append_attend_commit():
    """Window and full-attention layers of one sequence over 10 verify blocks: append the
    block's rows, attend (GPU) and check against the oracle on the true history, commit a
    random number of rows."""
    g = np.random.default_rng(9)
    R, W, hq, hkv, d, q_len = 2048, 512, 16, 4, 128, 16
    n_slots = n_table = 160                 # room for 10,240 positions
    kr = torch.zeros((R // CH, hkv, CH, d), dtype=torch.bfloat16, device="cuda")
    vr = torch.zeros((R // CH, hkv, d, CH), dtype=torch.bfloat16, device="cuda")
    kp = torch.zeros((n_slots, hkv, CH, d), dtype=torch.bfloat16, device="cuda")
    vp = torch.zeros((n_slots, hkv, d, CH), dtype=torch.bfloat16, device="cuda")
    table = torch.full((n_table,), -1, dtype=torch.int32, device="cuda")
    pager = rk.Pager(n_slots, n_table)
    hist_k = np.zeros((0, hkv, d), np.uint16)
    hist_v = np.zeros((0, hkv, d), np.uint16)

    def append(kb, vb):
        ctx = pager.ctx_len
        rk.verify_kv_append_ring(dev(kb), dev(vb), ctx, kr, vr)
        first, slots = pager.reserve(kb.shape[0])
        rk.verify_kv_append_paged(dev(kb), dev(vb), ctx, kp, vp, table, first, slots)

    # a committed prefix of 3,000 positions, appended in blocks of 1,000
    for _ in range(3):
        kb, vb = _bits(g, (1000, hkv, d)), _bits(g, (1000, hkv, d))
        append(kb, vb)
        pager.commit(1000)
        hist_k, hist_v = np.concatenate([hist_k, kb]), np.concatenate([hist_v, vb])
    for step in range(10):
        ctx = pager.ctx_len
        kb, vb = _bits(g, (q_len, hkv, d)), _bits(g, (q_len, hkv, d))
        q = _bits(g, (q_len, hq, d))
        append(kb, vb)
        rows_k, rows_v = np.concatenate([hist_k, kb]), np.concatenate([hist_v, vb])
        say(f"decode step {step}: ctx={ctx}")
        out, lse = rk.verify_attn_ring(dev(q), kr, vr, ctx, W)
        ref = oracle.attention_contiguous(q, rows_k, rows_v, ctx + q_len, window=W, dtype="bf16")
        assert np.abs(out.cpu().numpy() - ref[0]).max() <= TOL_BF16
        assert np.abs(lse.cpu().numpy() - ref[1]).max() <= TOL_LSE_BF16
        out, lse = rk.verify_attn_paged(dev(q), kp, vp, table, ctx + q_len)
        ref = oracle.attention_contiguous(q, rows_k, rows_v, ctx + q_len, dtype="bf16")
        assert np.abs(out.cpu().numpy() - ref[0]).max() <= TOL_BF16
        assert np.abs(lse.cpu().numpy() - ref[1]).max() <= TOL_LSE_BF16
        keep = int(g.integers(1, q_len + 1))
        pager.commit(keep)
        hist_k, hist_v = np.concatenate([hist_k, kb[:keep]]), np.concatenate([hist_v, vb[:keep]])
    assert pager.ctx_len == hist_k.shape[0]
