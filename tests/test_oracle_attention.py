"""Pins of the fp64 attention oracle against closed forms, invariants, brute force and a
library routine (CPU only)."""
import math

import numpy as np
import pytest
import torch

import oracle
from synth import (CHUNK, paged_store, ring_positions, ring_store, round_f32_to_bf16_bits,
                   contig_case, paged_case, ring_case)


def _rows(seed, n, hkv, d):
    g = np.random.default_rng(seed)
    return g.standard_normal((n, hkv, d)), g.standard_normal((n, hkv, d))


# --- bf16 decoding -------------------------------------------------------------------

def test_bf16_decode_known_patterns():
    bits = np.array([0x3F80, 0xC000, 0x0000, 0x8000, 0x0001, 0x7F7F, 0x3EAB, 0x4049], np.uint16)
    want = [1.0, -2.0, 0.0, -0.0, 2.0 ** -133, (2 - 2 ** -7) * 2.0 ** 127,
            0.333984375, 3.140625]
    got = oracle.bf16_to_f64(bits)
    assert got.dtype == np.float64
    assert list(got) == want
    assert math.copysign(1.0, got[3]) == -1.0


def test_bf16_rounding_of_inputs_is_nearest_even():
    # the generators' rounding, checked against the bf16 grid by hand
    x = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20, -3.0], np.float32)
    got = oracle.bf16_to_f64(round_f32_to_bf16_bits(x))
    assert list(got) == [1.0, 1.0 + 2 ** -6, 1.0 + 2 ** -7, -3.0]


# --- P1: Q = 0 -> every visible key has weight exactly 1 ----------------------------------

def _one_hot_rows(n, hkv, d):
    v = np.zeros((n, hkv, d))
    for j in range(n):
        for g in range(hkv):
            v[j, g, (j // CHUNK + 3 * g + j) % d] = 1.0
    return v


def _count_expect(q_pos, window, hkv, hq, d, n_keys_total):
    G = hq // hkv
    out = np.zeros((len(q_pos), hq, d))
    lse = np.zeros((len(q_pos), hq))
    for i, p in enumerate(q_pos):
        lo = max(0, p - window + 1) if window else 0
        n = p - lo + 1
        for h in range(hq):
            g = h // G
            for j in range(lo, p + 1):
                out[i, h, (j // CHUNK + 3 * g + j) % d] += 1.0 / n
            lse[i, h] = math.log(n)
    return out, lse


@pytest.mark.parametrize("ctx,q_len,window", [(300, 16, 0), (300, 16, 100), (1, 1, 0),
                                              (17, 17, 0), (700, 5, 512)])
def test_p1_zero_query_contiguous(ctx, q_len, window):
    hkv, hq, d = 2, 6, 8
    k, _ = _rows(1, ctx, hkv, d)
    v = _one_hot_rows(ctx, hkv, d)
    q = np.zeros((q_len, hq, d))
    out, lse = oracle.attention_contiguous(q, k, v, ctx, window=window, dtype="f64")
    q_pos = list(range(ctx - q_len, ctx))
    eo, el = _count_expect(q_pos, window, hkv, hq, d, ctx)
    np.testing.assert_allclose(out, eo, rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse, el, rtol=0, atol=1e-13)


def test_p1_window_has_exactly_w_keys():
    # the 512-token window includes the query's own position: lse = ln 512 exactly
    ctx, hkv, hq, d = 2000, 1, 1, 4
    k, v = _rows(2, ctx, hkv, d)
    q = np.zeros((16, hq, d))
    _, lse = oracle.attention_contiguous(q, k, v, ctx, window=512, dtype="f64")
    assert np.all(lse == math.log(512))


@pytest.mark.parametrize("pos0", [30000, 30720, 2040, 100])
def test_p1_zero_query_ring(pos0):
    hkv, hq, d, R, W, q_len = 2, 4, 8, 2048, 512, 16
    first, last = ring_positions(pos0, q_len, R)
    v = _one_hot_rows(last + 1, hkv, d)[first:]
    k, _ = _rows(3, last - first + 1, hkv, d)
    kr, vr = ring_store(k, v, first, R)
    q = np.zeros((q_len, hq, d))
    out, lse = oracle.attention_ring(q, kr, vr, pos0, pos0 % R, R, W, dtype="f64")
    eo, el = _count_expect(list(range(pos0, pos0 + q_len)), W, hkv, hq, d, last + 1)
    np.testing.assert_allclose(out, eo, rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse, el, rtol=0, atol=1e-13)


@pytest.mark.parametrize("ctx", [16, 17, 63, 64, 65, 1000])
def test_p1_zero_query_paged(ctx):
    hkv, hq, d, q_len = 2, 4, 8, 16
    v = _one_hot_rows(ctx, hkv, d)
    k, _ = _rows(4, ctx, hkv, d)
    nch = -(-ctx // CHUNK)
    pt = np.random.default_rng(ctx).permutation(nch + 3)[:nch]
    kp, vp = paged_store(k, v, pt, nch + 3)
    q = np.zeros((q_len, hq, d))
    out, lse = oracle.attention_paged(q, kp, vp, pt, ctx, dtype="f64")
    eo, el = _count_expect(list(range(ctx - q_len, ctx)), 0, hkv, hq, d, ctx)
    np.testing.assert_allclose(out, eo, rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse, el, rtol=0, atol=1e-13)


# --- P2: normalisation special cases ----------------------------------------------------

def test_p2_constant_values_and_single_key():
    hkv, hq, d, ctx = 2, 4, 8, 90
    k, _ = _rows(5, ctx, hkv, d)
    v = np.broadcast_to(np.linspace(-2, 3, d), (ctx, hkv, d)).copy()
    q = np.random.default_rng(6).standard_normal((8, hq, d)) * 3
    out, _ = oracle.attention_contiguous(q, k, v, ctx, dtype="f64")
    np.testing.assert_allclose(out, np.broadcast_to(v[0, 0], out.shape), rtol=0, atol=1e-14)
    # context of one token: the output is that token's value and lse its score
    out1, lse1 = oracle.attention_contiguous(q[:1], k[:1], v[:1] + k[:1], 1, dtype="f64")
    for h in range(hq):
        g = h // 2
        np.testing.assert_allclose(out1[0, h], (v[0] + k[0])[g], rtol=0, atol=1e-15)
        assert abs(lse1[0, h] - q[0, h] @ k[0, g] / math.sqrt(d)) < 1e-13


# --- P3: adding one vector to every key shifts every score of a row equally --------------

def test_p3_key_shift_invariance():
    hkv, hq, d, ctx = 2, 4, 16, 200
    k, v = _rows(7, ctx, hkv, d)
    q = np.random.default_rng(8).standard_normal((16, hq, d))
    u = np.random.default_rng(9).standard_normal((hkv, d)) * 4.0
    o1, l1 = oracle.attention_contiguous(q, k, v, ctx, window=64, dtype="f64")
    o2, l2 = oracle.attention_contiguous(q, k + u[None], v, ctx, window=64, dtype="f64")
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-12)
    G = hq // hkv
    shift = np.stack([q[:, h] @ u[h // G] for h in range(hq)], axis=1) / math.sqrt(d)
    np.testing.assert_allclose(l2 - l1, shift, rtol=0, atol=1e-11)


# --- P4: the library routine --------------------------------------------------------------

@pytest.mark.parametrize("ctx,q_len,hq,hkv,d,window", [(1024, 16, 8, 2, 64, 0),
                                                       (777, 16, 16, 4, 32, 512),
                                                       (40, 17, 4, 4, 8, 0),
                                                       (300, 3, 6, 1, 16, 7),
                                                       # prefill blocks: a whole prompt at
                                                       # once, and a long block after others
                                                       (1024, 1024, 8, 2, 16, 0),
                                                       (2000, 1024, 4, 1, 16, 512)])
def test_p4_matches_torch_sdpa(ctx, q_len, hq, hkv, d, window):
    k, v = _rows(10 + ctx, ctx, hkv, d)
    q = np.random.default_rng(11).standard_normal((q_len, hq, d))
    out, lse = oracle.attention_contiguous(q, k, v, ctx, window=window, dtype="f64")
    G = hq // hkv
    qt = torch.from_numpy(q).permute(1, 0, 2)[None]                     # [1][Hq][q][D]
    kt = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(G, 0)[None]
    vt = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(G, 0)[None]
    qp = torch.arange(ctx - q_len, ctx)[:, None]
    kp = torch.arange(ctx)[None, :]
    mask = kp <= qp
    if window:
        mask &= kp > qp - window
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask)
    np.testing.assert_allclose(out, ref[0].permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)
    # lse from the same library: logsumexp of the masked scaled scores
    s = (qt @ kt.transpose(-1, -2)) / math.sqrt(d)
    s = s.masked_fill(~mask, float("-inf"))
    np.testing.assert_allclose(lse, torch.logsumexp(s, -1)[0].T.numpy(), rtol=0, atol=1e-12)


# --- P5: tiny brute force with scalar loops -------------------------------------------------

@pytest.mark.parametrize("ctx,q_len,window", [(8, 3, 0), (8, 3, 2), (5, 1, 0), (3, 3, 0)])
def test_p5_scalar_brute_force(ctx, q_len, window):
    hq, hkv, d = 2, 1, 2
    g = np.random.default_rng(ctx * 10 + q_len)
    q = g.standard_normal((q_len, hq, d))
    k = g.standard_normal((ctx, hkv, d))
    v = g.standard_normal((ctx, hkv, d))
    out, lse = oracle.attention_contiguous(q, k, v, ctx, window=window, dtype="f64")
    sc = 1 / math.sqrt(d)
    for i in range(q_len):
        p = ctx - q_len + i
        for h in range(hq):
            js = [j for j in range(ctx) if j <= p and (window == 0 or j > p - window)]
            s = [sc * sum(q[i, h, t] * k[j, 0, t] for t in range(d)) for j in js]
            m = max(s)
            w = [math.exp(x - m) for x in s]
            l = math.fsum(w)
            for t in range(d):
                o = math.fsum(w[n] * v[js[n], 0, t] for n in range(len(js))) / l
                assert abs(out[i, h, t] - o) < 1e-14
            assert abs(lse[i, h] - (m + math.log(l))) < 1e-14


# --- P6: verify row i == single-token decode at context p_i + 1 -----------------------------

def test_p6_verify_row_equals_decode():
    c = contig_case(901, 0, 333, 16, 8, 2, 32, "f32")
    out, lse = oracle.attention_contiguous(c.q, c.k_rows, c.v_rows, c.ctx_len, dtype="f32")
    for i in range(16):
        p = c.ctx_len - 16 + i
        o1, l1 = oracle.attention_contiguous(c.q[i:i + 1], c.k_rows, c.v_rows, p + 1, dtype="f32")
        np.testing.assert_allclose(out[i], o1[0], rtol=0, atol=1e-14)
        np.testing.assert_allclose(lse[i], l1[0], rtol=0, atol=1e-13)


# --- P7: ring == contiguous sliding window -------------------------------------------------

@pytest.mark.parametrize("pos0", [30000, 30720, 2040, 100, 0, 2032])
def test_p7_ring_equals_contiguous_window(pos0):
    c = ring_case(902, 0, pos0, 16, 8, 2, 16, 2048, 512)
    out, lse = oracle.attention_ring(c.q, c.k_ring, c.v_ring, pos0, c.ring_head, 2048, 512)
    # the same rows laid out contiguously from position 0 (positions below the ring's
    # first are never visible, fill them with anything finite)
    n = c.ctx_len
    k = np.zeros((n, 2, 16), np.uint16)
    v = np.zeros((n, 2, 16), np.uint16)
    k[c.rows_first:] = c.k_rows
    v[c.rows_first:] = c.v_rows
    ro, rl = oracle.attention_contiguous(c.q, k, v, n, window=512, dtype="bf16")
    # same values, same order of the visible terms; only the zero terms differ in number
    np.testing.assert_allclose(out, ro, rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse, rl, rtol=0, atol=1e-14)


@pytest.mark.parametrize("pos0,q_len", [(30000, 1024), (0, 1024), (1023, 1537)])
def test_p7_ring_equals_contiguous_window_long_block(pos0, q_len):
    # a prefill block: window + q_len - 1 positions must fit the ring (1535 / 2048 at 1024)
    c = ring_case(905, 0, pos0, q_len, 4, 1, 16, 2048, 512)
    out, lse = oracle.attention_ring(c.q, c.k_ring, c.v_ring, pos0, c.ring_head, 2048, 512)
    n = c.ctx_len
    k = np.zeros((n, 1, 16), np.uint16)
    v = np.zeros((n, 1, 16), np.uint16)
    k[c.rows_first:] = c.k_rows
    v[c.rows_first:] = c.v_rows
    ro, rl = oracle.attention_contiguous(c.q, k, v, n, window=512, dtype="bf16")
    np.testing.assert_allclose(out, ro, rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse, rl, rtol=0, atol=1e-14)


def test_p7_ring_slot_rule_and_residency():
    c = ring_case(903, 0, 30000, 16, 4, 1, 8, 2048, 512)
    assert c.ring_head == 1328
    # the block's first query reads its own row at slot 1328 = chunk slot 20, offset 48
    np.testing.assert_array_equal(c.k_ring[20, 0, 48, :], c.k_rows[30000 - c.rows_first, 0])
    np.testing.assert_array_equal(c.v_ring[20, 0, :, 48], c.v_rows[30000 - c.rows_first, 0])
    with pytest.raises(ValueError):
        oracle.attention_ring(c.q, c.k_ring, c.v_ring, 30000, 1327, 2048, 512)
    small = ring_case(903, 1, 30000, 16, 4, 1, 8, 512, 512)
    with pytest.raises(ValueError):   # 527 positions do not fit in a 512-slot ring
        oracle.attention_ring(small.q, small.k_ring, small.v_ring, 30000, 30000 % 512, 512, 512)


# --- P8: paged == contiguous, for any permutation of the pool ------------------------------

@pytest.mark.parametrize("ctx", [8192, 1000, 65])
def test_p8_paged_equals_contiguous_any_permutation(ctx):
    outs = []
    for perm in ("identity", "seeded", "reversed"):
        c = paged_case(904, 0, ctx, 16, 8, 2, 32, n_slots=-(-ctx // 64) + 5, perm=perm)
        o, l = oracle.attention_paged(c.q, c.k_pool, c.v_pool, c.page_table, ctx)
        outs.append((o, l))
    ref = oracle.attention_contiguous(c.q, c.k_rows, c.v_rows, ctx, dtype="bf16")
    for o, l in outs:
        np.testing.assert_array_equal(o, ref[0])
        np.testing.assert_array_equal(l, ref[1])


def test_p8_paged_long_block_equals_contiguous():
    # a 1,000-query block over a permuted pool: every row equals contiguous attention
    c = paged_case(906, 0, 3000, 1000, 4, 2, 16, n_slots=60, perm="seeded")
    o, l = oracle.attention_paged(c.q, c.k_pool, c.v_pool, c.page_table, 3000)
    ro, rl = oracle.attention_contiguous(c.q, c.k_rows, c.v_rows, 3000, dtype="bf16")
    np.testing.assert_array_equal(o, ro)
    np.testing.assert_array_equal(l, rl)


def test_p8_store_layout_by_element():
    # the chunked layout, element by element: K(j)[g][d] at k_pool[pt[j//64], g, j%64, d],
    # V(j)[g][d] at v_pool[pt[j//64], g, d, j%64]
    ctx, hkv, d = 200, 3, 5
    k = np.arange(ctx * hkv * d, dtype=np.float64).reshape(ctx, hkv, d)
    v = -k
    pt = np.array([6, 1, 4, 0])
    kp, vp = paged_store(k, v, pt, 7)
    for j in range(ctx):
        for g in range(hkv):
            for t in range(d):
                assert kp[pt[j // 64], g, j % 64, t] == k[j, g, t]
                assert vp[pt[j // 64], g, t, j % 64] == v[j, g, t]
    assert np.isnan(kp[pt[3], 0, 8:, 0]).all()        # the tail of the last chunk is unset
    kr, vr = ring_store(k[:128], v[:128], 1990, 128)   # positions 1990..2117 in a 128-slot ring
    for j in range(1990, 2118):
        s = j % 128
        assert kr[s // 64, 1, s % 64, 2] == k[j - 1990, 1, 2]
        assert vr[s // 64, 2, 4, s % 64] == v[j - 1990, 2, 4]


# --- P9: split over key ranges + LSE merge == unsplit ---------------------------------------

@pytest.mark.parametrize("ctx", [16, 17, 63, 64, 65, 500, 8193, 8207])
def test_p9_split_merge_equals_unsplit(ctx):
    hkv, hq, d, q_len = 2, 8, 16, 16
    k, v = _rows(20 + ctx, ctx, hkv, d)
    q = np.random.default_rng(21).standard_normal((q_len, hq, d)) * 2
    whole = oracle.attention_contiguous(q, k, v, ctx, dtype="f64")
    q_pos = np.arange(ctx - q_len, ctx)
    g = np.random.default_rng(ctx)
    for n_parts in (1, 2, 5, 64):
        cuts = np.sort(g.choice(np.arange(1, ctx), size=min(n_parts - 1, ctx - 1), replace=False))
        bounds = [0, *cuts.tolist(), ctx]
        parts = []
        for a, b in zip(bounds[:-1], bounds[1:]):
            kp = np.arange(a, b)
            parts.append(oracle.attention_partial(q, lambda gg: k[a:b, gg], lambda gg: v[a:b, gg],
                                                  kp, q_pos, 0, 1 / math.sqrt(d), hkv))
        o, l = oracle.lse_merge(parts)
        np.testing.assert_allclose(o, whole[0], rtol=0, atol=1e-12)
        np.testing.assert_allclose(l, whole[1], rtol=0, atol=1e-12)


def test_p9_merge_skips_empty_parts():
    # a part in which a query sees no key carries lse = -inf and no weight
    q = np.zeros((1, 1, 2))
    k = np.zeros((3, 1, 2))
    v = np.array([[[1.0, 0.0]], [[0.0, 1.0]], [[5.0, 5.0]]])
    q_pos = np.array([1])
    p1 = oracle.attention_partial(q, lambda g: k[:2, g], lambda g: v[:2, g], [0, 1], q_pos, 0, 1.0, 1)
    p2 = oracle.attention_partial(q, lambda g: k[2:, g], lambda g: v[2:, g], [2], q_pos, 0, 1.0, 1)
    assert p2[1][0, 0] == -np.inf and np.all(p2[0] == 0)
    o, l = oracle.lse_merge([p1, p2])
    np.testing.assert_allclose(o[0, 0], [0.5, 0.5], atol=1e-15)
    assert abs(l[0, 0] - math.log(2)) < 1e-15


def test_p9_merge_at_logits_beyond_exp_range():
    """Scores in the thousands (lse 900 .. 2,500, where exp overflows float64): the merge still
    equals the unsplit softmax, and every part carries a real share of the weight."""
    hkv, hq, d, q_len, ctx = 2, 8, 16, 16, 700
    g = np.random.default_rng(31)
    k, v = g.standard_normal((ctx, hkv, d)), g.standard_normal((ctx, hkv, d))
    q = g.standard_normal((q_len, hq, d)) * 500
    whole = oracle.attention_contiguous(q, k, v, ctx, dtype="f64")
    assert whole[1].min() > 710                 # exp(lse) is not representable
    q_pos = np.arange(ctx - q_len, ctx)
    bounds = [0, 100, 333, 650, ctx]
    parts = [oracle.attention_partial(q, lambda gg, a=a, b=b: k[a:b, gg],
                                      lambda gg, a=a, b=b: v[a:b, gg], np.arange(a, b), q_pos,
                                      0, 1 / math.sqrt(d), hkv)
             for a, b in zip(bounds[:-1], bounds[1:])]
    assert all(np.exp(p[1] - whole[1]).mean() > 0.05 for p in parts)
    o, l = oracle.lse_merge(parts)
    np.testing.assert_allclose(o, whole[0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(l, whole[1], rtol=1e-14, atol=0)
