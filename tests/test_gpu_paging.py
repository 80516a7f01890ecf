"""GPU parity of host paging (HIP kernels and copy engines through the C interface): chunks
paged out to pinned host memory and back in bit-exact, attention over the resident subset of the
pool against the fp64 oracle, and a sequence whose context outgrows the pool, kept going by
paging its oldest chunks out."""
import numpy as np
import pytest
import torch

import oracle
import ring_kv_amd as rk
from gpu_util import assert_attn_close, dev, say
from synth import paged_case, round_f32_to_bf16_bits

pytestmark = pytest.mark.gpu
CH = 64


def _bits(g, shape):
    return round_f32_to_bf16_bits(g.standard_normal(shape).astype(np.float32))


def _host(t):
    return t.view(torch.int16).numpy().view(np.uint16) if not t.is_cuda else \
        t.view(torch.int16).cpu().numpy().view(np.uint16)


def _pinned(shape):
    return torch.zeros(shape, dtype=torch.bfloat16, pin_memory=True)


@pytest.mark.parametrize("pattern,pinned", [("runs", True), ("mixed", True), ("scattered", True),
                                            ("scattered", False)])
def test_page_out_in_round_trip_bit_exact(pattern, pinned):
    """300 chunks (two batches) out to a host store and back into other slots: long runs of chunk
    ids go through the copy engines, scattered ids through the direct kernel (pinned stores) or
    one copy per run (a pageable store)."""
    g = np.random.default_rng(61)
    n_slots, hkv, d, n_host = 400, 4, 128, 500
    kp, vp = _bits(g, (n_slots, hkv, CH, d)), _bits(g, (n_slots, hkv, d, CH))
    kd, vd = dev(kp), dev(vp)
    make = _pinned if pinned else (lambda sh: torch.zeros(sh, dtype=torch.bfloat16))
    kh, vh = make((n_host, hkv, CH, d)), make((n_host, hkv, d, CH))
    if pattern == "runs":
        ids = list(range(10, 160)) + list(range(300, 450))
    elif pattern == "mixed":
        ids = list(range(10, 150)) + list(range(300, 380)) + \
            [int(c) for c in g.choice(np.arange(400, 500), 80, replace=False)]
    else:
        ids = [int(c) for c in g.choice(n_host, 300, replace=False)]
    slots = [int(s) for s in g.permutation(n_slots)[:len(ids)]]
    say(f"page out {len(ids)} chunks ({pattern}, {'pinned' if pinned else 'pageable'})")
    rk.kv_page_out(kd, vd, slots, ids, kh, vh)
    torch.cuda.synchronize()
    khn, vhn = _host(kh), _host(vh)
    for c, s in zip(ids, slots):
        np.testing.assert_array_equal(khn[c], kp[s])
        np.testing.assert_array_equal(vhn[c], vp[s])
    untouched = sorted(set(range(n_host)) - set(ids))
    assert not np.any(khn[untouched]) and not np.any(vhn[untouched])
    # back into a fresh pool at other slots: the same bits there
    k2 = torch.zeros_like(kd)
    v2 = torch.zeros_like(vd)
    new = [int(s) for s in g.permutation(n_slots)[:len(ids)]]
    say("page in")
    rk.kv_page_in(kh, vh, ids, new, k2, v2)
    k2n, v2n = _host(k2), _host(v2)
    for s_old, s_new in zip(slots, new):
        np.testing.assert_array_equal(k2n[s_new], kp[s_old])
        np.testing.assert_array_equal(v2n[s_new], vp[s_old])
    rest = sorted(set(range(n_slots)) - set(new))
    assert not np.any(k2n[rest])


@pytest.mark.parametrize("ctx,q_len,n_keep", [(20000, 16, 100), (9216, 1024, 40), (4096, 16, 0)])
def test_resident_attention_matches_oracle(ctx, q_len, n_keep):
    c = paged_case(62, q_len, ctx, q_len, 16, 4, 128)
    nch = -(-ctx // CH)
    first = (ctx - q_len) // CH
    g = np.random.default_rng(ctx)
    keep = sorted(int(x) for x in g.choice(first, size=min(n_keep, first), replace=False))
    ids = keep + list(range(first, nch))
    slots = [int(c.page_table[i]) for i in ids]
    say(f"resident attention ctx={ctx} q_len={q_len}: {len(ids)} of {nch} chunks")
    q, kp, vp = dev(c.q), dev(c.k_pool), dev(c.v_pool)
    out, lse = rk.verify_attn_paged_resident(q, kp, vp, dev(np.array(slots, np.int32)), ids, ctx)
    torch.cuda.synchronize()
    want = oracle.attention_resident(c.q, c.k_pool, c.v_pool, ids, slots, ctx)
    assert_attn_close((out.cpu().numpy(), lse.cpu().numpy()), want, "bf16", f"resident {ctx}")


def test_all_resident_equals_the_dense_call():
    c = paged_case(63, 0, 8192, 16, 16, 4, 128)
    q, kp, vp, pt = dev(c.q), dev(c.k_pool), dev(c.v_pool), dev(c.page_table)
    say("all chunks resident")
    o1, l1 = rk.verify_attn_paged(q, kp, vp, pt, 8192)
    o2, l2 = rk.verify_attn_paged_resident(q, kp, vp, pt, list(range(128)), 8192)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_context_larger_than_the_pool():
    """A 6,000-token context through a 48-slot pool (3,072 positions): blocks of 1,024 (then
    verify blocks of 16) are appended and attended over the resident chunks; before each block
    the oldest whole chunks are paged out to pinned host memory so that the block fits.  Every
    attention matches the oracle over the same resident subset, every paged-out chunk holds its
    true rows on the host, and paging chunks back in restores them bit-exact."""
    g = np.random.default_rng(64)
    hq, hkv, d = 16, 4, 128
    n_slots, n_table = 48, 120
    kp = torch.zeros((n_slots, hkv, CH, d), dtype=torch.bfloat16, device="cuda")
    vp = torch.zeros((n_slots, hkv, d, CH), dtype=torch.bfloat16, device="cuda")
    table = torch.full((n_table,), -1, dtype=torch.int32, device="cuda")
    kh, vh = _pinned((n_table, hkv, CH, d)), _pinned((n_table, hkv, d, CH))
    pager = rk.Pager(n_slots, n_table)
    hist_k = np.zeros((0, hkv, d), np.uint16)
    hist_v = np.zeros((0, hkv, d), np.uint16)
    blocks = [1024] * 5 + [16] * 6 + [880]
    for step, n in enumerate(blocks):
        ctx = pager.ctx_len
        need = -(-(ctx + n) // CH) - (-(-ctx // CH))
        if pager.free_slots < need:
            ids, _ = pager.resident()
            old = [c for c in ids if c < ctx // CH][:need - pager.free_slots + 2]
            slots = pager.evict(old)
            say(f"step {step}: page out chunks {old[0]}..{old[-1]} ({len(old)})")
            rk.kv_page_out(kp, vp, slots, old, kh, vh)
        kb, vb, q = _bits(g, (n, hkv, d)), _bits(g, (n, hkv, d)), _bits(g, (n, hq, d))
        first, new = pager.reserve(n)
        rk.verify_kv_append_paged(dev(kb), dev(vb), ctx, kp, vp, table, first, new)
        hist_k, hist_v = np.concatenate([hist_k, kb]), np.concatenate([hist_v, vb])
        ids, slots = pager.resident()
        say(f"step {step}: block of {n} at {ctx}, {len(ids)} chunks resident")
        out, lse = rk.verify_attn_paged_resident(dev(q), kp, vp, dev(np.array(slots, np.int32)),
                                                 ids, ctx + n)
        torch.cuda.synchronize()
        # the oracle over the same chunks' positions, read from the true history
        pos = np.concatenate([np.arange(c * CH, min(c * CH + CH, ctx + n)) for c in ids])
        want = oracle.attend_rows(oracle.bf16_to_f64(q),
                                  lambda gg: oracle.bf16_to_f64(hist_k[pos, gg]),
                                  lambda gg: oracle.bf16_to_f64(hist_v[pos, gg]), pos,
                                  ctx + np.arange(n), 0, 1 / np.sqrt(d), hkv)
        assert_attn_close((out.cpu().numpy(), lse.cpu().numpy()), want, "bf16", f"step {step}")
        pager.commit(n)
    # every paged-out chunk holds its true rows on the host
    tab = pager.table()
    out_ids = [c for c, s in enumerate(tab) if s == -2]
    assert len(out_ids) > 40
    khn, vhn = _host(kh), _host(vh)
    for c in out_ids:
        np.testing.assert_array_equal(khn[c], hist_k[c * CH:(c + 1) * CH].transpose(1, 0, 2))
        np.testing.assert_array_equal(vhn[c], hist_v[c * CH:(c + 1) * CH].transpose(1, 2, 0))
    # page the first chunks back in (after paging others out to make room): bit-exact
    ids, _ = pager.resident()
    make_room = [c for c in ids if c < pager.ctx_len // CH][:10]
    rk.kv_page_out(kp, vp, pager.evict(make_room), make_room, kh, vh)
    back = out_ids[:10]
    slots = pager.restore(back)
    say(f"page in chunks {back}")
    rk.kv_page_in(kh, vh, back, slots, kp, vp)
    kpn, vpn = _host(kp), _host(vp)
    for c, s in zip(back, slots):
        np.testing.assert_array_equal(kpn[s], hist_k[c * CH:(c + 1) * CH].transpose(1, 0, 2))
        np.testing.assert_array_equal(vpn[s], hist_v[c * CH:(c + 1) * CH].transpose(1, 2, 0))
