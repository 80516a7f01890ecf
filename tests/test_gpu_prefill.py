"""GPU parity of batched prefill attention (blocks of hundreds to thousands of queries through the
pool and the ring; the matrix-core kernel behind the same C entry points) against the fp64 oracle:
the named 1,024-token workloads, exact key coverage, ragged blocks and tiles, splits, shapes, table
faults, the two-phase form, and a prompt prefilled block by block through the append path."""
import math

import numpy as np
import pytest
import torch

import oracle
import ring_kv_amd as rk
from synth import paged_case, paged_store, ring_case, ring_positions, ring_store, workload
from synth import round_f32_to_bf16_bits
from gpu_util import TOL_BF16, TOL_LSE_BF16, assert_attn_close, dev, run_gpu, run_oracle, say

pytestmark = pytest.mark.gpu


# ---- the named prefill workloads -------------------------------------------------------------

def test_prefill_pool_8k_splits_and_determinism():
    """Splits 1 and 3 leave 256-row tiles short of the chip: 1 runs 64-row tiles (two row groups,
    two waves per row group, one per half of each chunk's keys; that grid of 256 workgroups still
    fits one round) and 3 runs 128-row tiles (its 64-row grid would take more than one round);
    0 (auto, 4) and 7 run 256-row tiles."""
    c, _ = workload("prefill_pool_8k")
    say("prefill_pool_8k: oracle")
    ref = run_oracle(c)
    first = None
    for s in (0, 1, 3, 7):
        say(f"prefill_pool_8k splits={s}")
        got = run_gpu(c, num_splits=s)
        assert_attn_close(got, ref, "bf16", f"prefill_pool_8k S={s}")
        if s == 0:
            first = got
    again = run_gpu(c)
    np.testing.assert_array_equal(again[0], first[0])
    np.testing.assert_array_equal(again[1], first[1])


def test_prefill_pool_permutation_invariance():
    c, _ = workload("prefill_pool_8k")
    got = run_gpu(c)
    for perm in ("identity", "reversed"):
        say(f"prefill pool perm={perm}")
        c2 = paged_case(6, 0, 9216, 1024, 16, 4, 128, n_slots=160, perm=perm)
        np.testing.assert_array_equal(c2.k_rows, c.k_rows)
        g2 = run_gpu(c2)
        np.testing.assert_array_equal(g2[0], got[0])
        np.testing.assert_array_equal(g2[1], got[1])


def test_prefill_ring_w512():
    c, _ = workload("prefill_ring_w512")
    say("prefill_ring_w512: oracle")
    ref = run_oracle(c)
    for s in (0, 2, 5):
        say(f"prefill_ring_w512 splits={s}")
        assert_attn_close(run_gpu(c, num_splits=s), ref, "bf16", f"prefill ring S={s}")


def test_prefill_pool_131k_sampled_rows():
    """Full size: every row of the block is computed; a quarter of its rows are checked against
    the oracle: four runs of 64 consecutive rows (the block's first and last, one across the
    256-row tile edge at 256, one inside a tile), each as a 64-query block at its own context, and
    single rows at the other tile edges as single-token decodes at their own context (the
    verify/decode equivalence)."""
    c, _ = workload("prefill_pool_131k")
    say("prefill_pool_131k: gpu")
    out, lse = run_gpu(c)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
    p0 = c.ctx_len - c.q_len
    for a in (0, 224, 600, 960):
        say(f"prefill_pool_131k: oracle rows {a}..{a + 63}")
        want = oracle.attention_paged(c.q[a:a + 64], c.k_pool, c.v_pool, c.page_table, p0 + a + 64)
        assert_attn_close((out[a:a + 64], lse[a:a + 64]), want, "bf16", f"131k rows {a}..{a + 63}")
    for i in (511, 512, 767, 768):
        want = oracle.attention_paged(c.q[i:i + 1], c.k_pool, c.v_pool, c.page_table, p0 + i + 1)
        assert_attn_close((out[i:i + 1], lse[i:i + 1]), want, "bf16", f"131k row {i}")


@pytest.mark.parametrize("store,q_len,hq,hkv,d", [("paged", 4096, 16, 4, 128),
                                                  ("ring", 4096, 16, 4, 128),
                                                  ("paged", 16384, 2, 2, 64)])
def test_prefill_max_rows_sampled(store, q_len, hq, hkv, d):
    """The largest block one call may carry, RKV_MAX_ROWS = 16,384 rows per KV head (4,096
    queries x 4 query heads per KV head: 256-row tiles; or 16,384 queries without grouping on 2
    KV heads: 128-row tiles), over the pool and over a ring that holds every query's window.
    Every row is computed; sampled rows (both ends, tile and chunk edges) are checked against the
    oracle as single-token decodes at their own positions."""
    if store == "paged":
        c = paged_case(926, q_len, q_len + 904, q_len, hq, hkv, d, keep_rows=False)
        p0 = c.ctx_len - q_len
    else:
        R, W = 4608, 512                      # R = W + q_len: the smallest multiple of 64 that holds
        c = ring_case(927, q_len, 70000, q_len, hq, hkv, d, R, W)
        p0 = c.pos0
    assert q_len * (hq // hkv) == 16384
    rows = (0, 1, 31, 32, 63, 64, 127, 128, 2047, 2048, q_len - 65, q_len - 2, q_len - 1)
    want = {}
    for i in rows:
        if store == "paged":
            want[i] = oracle.attention_paged(c.q[i:i + 1], c.k_pool, c.v_pool, c.page_table,
                                             p0 + i + 1)
        else:
            want[i] = oracle.attention_ring(c.q[i:i + 1], c.k_ring, c.v_ring, p0 + i,
                                            (p0 + i) % c.ring_size, c.ring_size, c.window)
    # auto splits, and one split (which leaves the G = 1 block on 128-row tiles)
    for splits in (0, 1):
        say(f"prefill max rows {store} q_len={q_len} hq={hq} hkv={hkv} d={d} splits={splits}")
        out, lse = run_gpu(c, num_splits=splits)
        assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
        for i in rows:
            assert_attn_close((out[i:i + 1], lse[i:i + 1]), want[i], "bf16",
                              f"max rows {store} splits={splits} row {i}")

# ---- exact coverage: zero Q, one-hot V -> each row's output counts its visible keys -------------

def _one_hot_v(n, first, hkv, d):
    v = np.zeros((n, hkv, d), np.float32)
    for g in range(hkv):
        pos = np.arange(first, first + n)
        v[np.arange(n), g, (pos // 64 + 3 * g + pos) % d] = 1.0
    return round_f32_to_bf16_bits(v)


def _count(q_pos, window, hkv, d, G):
    out = np.zeros((len(q_pos), hkv * G, d))
    lse = np.zeros((len(q_pos), hkv * G))
    for i, p in enumerate(q_pos):
        lo = max(0, p - window + 1) if window else 0
        j = np.arange(lo, p + 1)
        for g in range(hkv):
            row = np.bincount((j // 64 + 3 * g + j) % d, minlength=d) / len(j)
            out[i, g * G:(g + 1) * G] = row
        lse[i] = math.log(len(j))
    return out, lse


@pytest.mark.parametrize("ctx,q_len,splits", [(1024, 1024, 0), (9216, 1024, 0), (9216, 1024, 5),
                                              (5000, 1000, 0), (377, 300, 2)])
def test_prefill_exact_coverage_paged(ctx, q_len, splits):
    hq, hkv, d = 16, 4, 128
    nch = -(-ctx // 64)
    pt = np.random.default_rng(ctx).permutation(nch).astype(np.int32)
    kp, vp = paged_store(np.zeros((ctx, hkv, d), np.uint16), _one_hot_v(ctx, 0, hkv, d), pt, nch)
    say(f"prefill coverage paged ctx={ctx} q_len={q_len} splits={splits}")
    out, lse = rk.verify_attn_paged(dev(np.zeros((q_len, hq, d), np.uint16)), dev(kp), dev(vp),
                                    dev(pt), ctx, num_splits=splits)
    eo, el = _count(range(ctx - q_len, ctx), 0, hkv, d, hq // hkv)
    np.testing.assert_allclose(out.cpu().numpy(), eo, rtol=0, atol=2e-6)
    np.testing.assert_allclose(lse.cpu().numpy(), el, rtol=0, atol=2e-6)


@pytest.mark.parametrize("pos0,q_len", [(30000, 1024), (0, 1024), (100, 1024), (2048, 1537)])
def test_prefill_exact_coverage_ring(pos0, q_len):
    hq, hkv, d, R, W = 16, 4, 128, 2048, 512
    first, last = ring_positions(pos0, q_len, R)
    n = last - first + 1
    kr, vr = ring_store(np.zeros((n, hkv, d), np.uint16), _one_hot_v(n, first, hkv, d), first, R)
    say(f"prefill coverage ring pos0={pos0} q_len={q_len}")
    out, lse = rk.verify_attn_ring(dev(np.zeros((q_len, hq, d), np.uint16)), dev(kr), dev(vr),
                                   pos0, W)
    eo, el = _count(range(pos0, pos0 + q_len), W, hkv, d, hq // hkv)
    np.testing.assert_allclose(out.cpu().numpy(), eo, rtol=0, atol=2e-6)
    np.testing.assert_allclose(lse.cpu().numpy(), el, rtol=0, atol=2e-6)


# ---- ragged blocks, shapes, ring positions ----------------------------------------------------------

@pytest.mark.parametrize("ctx,q_len", [(65, 65), (1000, 1000), (3000, 700), (4161, 1025)])
def test_prefill_paged_ragged(ctx, q_len):
    c = paged_case(920, ctx, ctx, q_len, 16, 4, 128, n_slots=-(-ctx // 64) + 5)
    ref = run_oracle(c)
    for s in (0, 1, 3):
        say(f"prefill paged ctx={ctx} q_len={q_len} splits={s}")
        assert_attn_close(run_gpu(c, num_splits=s), ref, "bf16", f"prefill ctx={ctx} S={s}")


@pytest.mark.parametrize("q_len,hq,hkv,d", [(512, 8, 8, 128), (256, 32, 4, 128), (1024, 16, 4, 64),
                                            (300, 6, 2, 64)])
def test_prefill_paged_shapes(q_len, hq, hkv, d):
    c = paged_case(921, q_len + hq, 2500 + q_len, q_len, hq, hkv, d, n_slots=60)
    say(f"prefill paged shape q_len={q_len} hq={hq} hkv={hkv} d={d}")
    assert_attn_close(run_gpu(c), run_oracle(c), "bf16", f"prefill shape {q_len},{hq},{hkv},{d}")


@pytest.mark.parametrize("pos0,q_len,R,W", [(0, 1024, 2048, 512), (100, 1024, 2048, 512),
                                            (2040, 777, 2048, 512), (5000, 600, 640, 41),
                                            (70000, 1024, 1536, 513)])
def test_prefill_ring_positions(pos0, q_len, R, W):
    c = ring_case(922, pos0, pos0, q_len, 16, 4, 128, R, W)
    say(f"prefill ring pos0={pos0} q_len={q_len} R={R} W={W}")
    assert_attn_close(run_gpu(c), run_oracle(c), "bf16", f"prefill ring pos0={pos0}")


def test_prefill_ring_d64():
    c = ring_case(923, 0, 9000, 1024, 16, 4, 64, 2048, 512)
    say("prefill ring d=64")
    assert_attn_close(run_gpu(c), run_oracle(c), "bf16", "prefill ring d=64")


# ---- table faults, two-phase form -------------------------------------------------------------------

def test_prefill_out_of_range_entry_contributes_nothing():
    c = paged_case(924, 0, 4096, 1024, 16, 4, 128, n_slots=64)
    pt = c.page_table.copy()
    pt[5] = 64
    pt[60] = -3          # inside the block's own chunks
    say("prefill paged with out-of-range table entries")
    out, lse = rk.verify_attn_paged(dev(c.q), dev(c.k_pool), dev(c.v_pool), dev(pt), 4096)
    keep = np.array([j for j in range(4096) if j // 64 not in (5, 60)])
    kg, vg = oracle.gather_paged(c.k_pool, c.v_pool, c.page_table, keep)
    ref = oracle.attend_rows(oracle.to_f64(c.q, "bf16"), lambda g: oracle.to_f64(kg(g), "bf16"),
                             lambda g: oracle.to_f64(vg(g), "bf16"), keep, np.arange(3072, 4096),
                             0, 1 / math.sqrt(128), 4)
    torch.cuda.synchronize()
    o, l = out.cpu().numpy(), lse.cpu().numpy()
    # rows whose every visible key is gone (none here) would be 0 / -inf; all others compare
    assert_attn_close((o, l), ref, "bf16", "prefill bad entries")


def test_prefill_two_phase_equals_direct():
    c, _ = workload("prefill_pool_8k")
    q, kp, vp, pt = dev(c.q), dev(c.k_pool), dev(c.v_pool), dev(c.page_table)
    say("prefill two-phase")
    o1, l1 = rk.verify_attn_paged(q, kp, vp, pt, c.ctx_len, num_splits=3)
    po, pl = rk.verify_attn_paged_partial(q, kp, vp, pt, c.ctx_len, 3)
    o2, l2 = rk.attn_merge_partials(po, pl, c.q_len, c.n_q_heads)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_prefill_partials_of_each_split():
    """A block that starts the context: 4 splits of 4 chunks; the early rows see nothing of the
    later splits (lse -inf, zero output), the others match the oracle over the split's keys."""
    c = paged_case(925, 0, 1024, 1024, 16, 4, 128)
    q, kp, vp, pt = dev(c.q), dev(c.k_pool), dev(c.v_pool), dev(c.page_table)
    say("prefill partials per split")
    po, pl = rk.verify_attn_paged_partial(q, kp, vp, pt, 1024, 4)
    torch.cuda.synchronize()
    pon, pln = po.cpu().numpy(), pl.cpu().numpy()
    qf = oracle.to_f64(c.q, "bf16")
    for s in range(4):
        keys = np.arange(s * 256, (s + 1) * 256)
        kg, vg = oracle.gather_paged(c.k_pool, c.v_pool, c.page_table, keys)
        o, l = oracle.attend_rows(qf, lambda g: oracle.to_f64(kg(g), "bf16"),
                                  lambda g: oracle.to_f64(vg(g), "bf16"), keys, np.arange(1024),
                                  0, 1 / math.sqrt(128), 4)
        for g in range(4):
            rows = np.arange(4096)
            i, h = rows // 4, g * 4 + rows % 4
            seen = np.isfinite(l[i, h])
            assert np.all(pln[g, s, ~seen] == -np.inf) and np.all(pon[g, s, ~seen] == 0)
            assert np.abs(pon[g, s, seen] - o[i[seen], h[seen]]).max() <= TOL_BF16
            assert np.abs(pln[g, s, seen] - l[i[seen], h[seen]]).max() <= TOL_LSE_BF16


# ---- a prompt prefilled block by block --------------------------------------------------------------

def test_prompt_prefill_by_blocks_append_and_attend():
    """A 2,500-token prompt in blocks of 1,024, 1,024 and 452: each block's rows are appended to
    the ring and the pool, then its attention is read from both and checked against the oracle
    on the true history (window layer and full layer)."""
    g = np.random.default_rng(31)
    R, W, hq, hkv, d = 2048, 512, 16, 4, 128
    n_slots = n_table = 48
    kr = torch.zeros((R // 64, hkv, 64, d), dtype=torch.bfloat16, device="cuda")
    vr = torch.zeros((R // 64, hkv, d, 64), dtype=torch.bfloat16, device="cuda")
    kp = torch.zeros((n_slots, hkv, 64, d), dtype=torch.bfloat16, device="cuda")
    vp = torch.zeros((n_slots, hkv, d, 64), dtype=torch.bfloat16, device="cuda")
    table = torch.full((n_table,), -1, dtype=torch.int32, device="cuda")
    pager = rk.Pager(n_slots, n_table)
    hist_k = np.zeros((0, hkv, d), np.uint16)
    hist_v = np.zeros((0, hkv, d), np.uint16)

    def bits(shape):
        return round_f32_to_bf16_bits(g.standard_normal(shape).astype(np.float32))

    for n in (1024, 1024, 452):
        ctx = pager.ctx_len
        kb, vb, q = bits((n, hkv, d)), bits((n, hkv, d)), bits((n, hq, d))
        rk.verify_kv_append_ring(dev(kb), dev(vb), ctx, kr, vr)
        first, slots = pager.reserve(n)
        rk.verify_kv_append_paged(dev(kb), dev(vb), ctx, kp, vp, table, first, slots)
        hist_k, hist_v = np.concatenate([hist_k, kb]), np.concatenate([hist_v, vb])
        say(f"prompt block at {ctx}: {n} tokens")
        out, lse = rk.verify_attn_ring(dev(q), kr, vr, ctx, W)
        ref = oracle.attention_contiguous(q, hist_k, hist_v, ctx + n, window=W, dtype="bf16")
        assert_attn_close((out.cpu().numpy(), lse.cpu().numpy()), ref, "bf16", f"ring @{ctx}")
        out, lse = rk.verify_attn_paged(dev(q), kp, vp, table, ctx + n)
        ref = oracle.attention_contiguous(q, hist_k, hist_v, ctx + n, dtype="bf16")
        assert_attn_close((out.cpu().numpy(), lse.cpu().numpy()), ref, "bf16", f"pool @{ctx}")
        pager.commit(n)
    assert pager.ctx_len == 2500
