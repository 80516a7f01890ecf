"""Plant plausible mistakes in copies of the oracle's attention core (CPU only) and check
that the pins catch each of them: the pins are not vacuous."""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import attention as A


def _mutant(kind):
    def attend_rows(q, k_of_head, v_of_head, key_pos, q_pos, window, scale, n_kv_heads):
        q = np.asarray(q, dtype=np.float64)
        q_len, hq, d = q.shape
        G = hq // n_kv_heads
        key_pos = np.asarray(key_pos)
        q_pos = np.asarray(q_pos)
        w_eff = window + 1 if (kind == "window_off_by_one" and window) else window
        lo = np.array([A.key_bounds(int(p), w_eff)[0] for p in q_pos])
        hi = q_pos - 1 if kind == "strict_causal" else q_pos
        visible = (key_pos[None, :] >= lo[:, None]) & (key_pos[None, :] <= hi[:, None])
        out = np.zeros((q_len, hq, d))
        lse = np.full((q_len, hq), -np.inf)
        sc = 1.0 if kind == "no_scale" else scale
        for h in range(hq):
            g = h % n_kv_heads if kind == "gqa_modulo" else h // G
            Kg, Vg = k_of_head(g), v_of_head(g)
            s = sc * (q[:, h, :] @ Kg.T)
            s = np.where(visible, s, -np.inf)
            m = s.max(axis=1)
            has = np.isfinite(m)
            w = np.exp(s - np.where(has, m, 0.0)[:, None])
            l = w.sum(axis=1)
            if kind == "no_normalise":
                l = np.ones_like(l)
            o = w @ Vg
            out[has, h] = o[has] / l[has, None]
            lse[has, h] = m[has] + np.log(l[has])
        return out, lse
    return attend_rows


def _sdpa_pin(ctx=300, q_len=16, hq=8, hkv=2, d=16, window=64):
    g = np.random.default_rng(1)
    k, v = g.standard_normal((ctx, hkv, d)), g.standard_normal((ctx, hkv, d))
    q = g.standard_normal((q_len, hq, d))
    out, _ = oracle.attention_contiguous(q, k, v, ctx, window=window, dtype="f64")
    G = hq // hkv
    qt = torch.from_numpy(q).permute(1, 0, 2)[None]
    kt = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(G, 0)[None]
    vt = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(G, 0)[None]
    qp, kp = torch.arange(ctx - q_len, ctx)[:, None], torch.arange(ctx)[None, :]
    mask = (kp <= qp) & (kp > qp - window)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask)
    return np.abs(out - ref[0].permute(1, 0, 2).numpy()).max() < 1e-12


def _count_pin():
    ctx = 2000
    k = np.random.default_rng(2).standard_normal((ctx, 1, 4))
    _, lse = oracle.attention_contiguous(np.zeros((16, 1, 4)), k, k, ctx, window=512, dtype="f64")
    return bool(np.all(lse == math.log(512)))


def _ring_pin():
    from synth import ring_case
    c = ring_case(77, 0, 30720, 16, 4, 2, 8, 2048, 512)
    out, _ = oracle.attention_ring(c.q, c.k_ring, c.v_ring, c.pos0, c.ring_head, 2048, 512)
    n = c.ctx_len
    k = np.zeros((n, 2, 8), np.uint16)
    v = np.zeros((n, 2, 8), np.uint16)
    k[c.rows_first:], v[c.rows_first:] = c.k_rows, c.v_rows
    ro, _ = oracle.attention_contiguous(c.q, k, v, n, window=512, dtype="bf16")
    return np.abs(out - ro).max() < 1e-14


def test_unmutated_oracle_passes_the_pins():
    assert _sdpa_pin() and _count_pin() and _ring_pin()


@pytest.mark.parametrize("kind", ["window_off_by_one", "strict_causal", "no_scale",
                                  "gqa_modulo", "no_normalise"])
def test_each_planted_mistake_is_caught(kind, monkeypatch):
    monkeypatch.setattr(A, "attend_rows", _mutant(kind))
    assert not (_sdpa_pin() and _count_pin())


def test_planted_ring_slot_mistake_is_caught(monkeypatch):
    real = A.gather_ring

    def shifted(k_ring, v_ring, positions, ring_size, chunk=64):
        return real(k_ring, v_ring, np.asarray(positions) + 1, ring_size, chunk)
    monkeypatch.setattr(A, "gather_ring", shifted)
    assert not _ring_pin()


def test_planted_v_transpose_mistake_is_caught(monkeypatch):
    from synth import paged_case

    def wrong(k_pool, v_pool, page_table, positions, chunk=64):
        positions = np.asarray(positions)
        slot = np.asarray(page_table)[positions // chunk]
        off = positions % chunk
        # reads V as if it were stored key-major like K
        return (lambda g: np.asarray(k_pool)[slot, g, off, :],
                lambda g: np.asarray(v_pool).reshape(v_pool.shape[0], v_pool.shape[1], chunk, -1)[slot, g, off, :])
    c = paged_case(78, 0, 500, 16, 4, 2, 64)
    ref = oracle.attention_contiguous(c.q, c.k_rows, c.v_rows, 500, dtype="bf16")
    monkeypatch.setattr(A, "gather_paged", wrong)
    o, _ = oracle.attention_paged(c.q, c.k_pool, c.v_pool, c.page_table, 500)
    assert not (np.abs(o - ref[0]).max() <= 1e-3)   # wrong values or NaN from unset slots


# --- the cache oracle: planted mistakes in copies of the append / commit rules --------------

def _cache_mutant(kind):
    """(append_ring, append_paged, PagerModel) with one planted mistake."""
    from oracle import cache as C

    def append_ring(k_ring, v_ring, k_new, v_new, pos_first):
        k, v = np.array(k_ring, copy=True), np.array(v_ring, copy=True)
        ring = k.shape[0] * C.CHUNK
        for i in range(k_new.shape[0]):
            s = (pos_first + i + (1 if kind == "ring_slot_shift" else 0)) % ring
            for g in range(k_new.shape[1]):
                k[s // C.CHUNK, g, s % C.CHUNK, :] = k_new[i, g, :]
                if kind == "v_key_major":
                    v[s // C.CHUNK, g, s % C.CHUNK, :] = v_new[i, g, :]
                else:
                    v[s // C.CHUNK, g, :, s % C.CHUNK] = v_new[i, g, :]
        return k, v

    class Pager(C.PagerModel):
        def commit(self, n_keep):
            if kind != "free_committed_chunk":
                return super().commit(n_keep)
            _, first, k = self.pending
            self.ctx += n_keep
            keep = self.ctx // C.CHUNK                 # floor: frees a partly committed chunk
            for c in range(first + k - 1, first - 1, -1):
                if c < keep:
                    break
                self.free.append(self.table[c])
                self.table[c] = -1
            self.pending = None

    return append_ring, C.append_paged, Pager


@pytest.mark.parametrize("kind", ["ring_slot_shift", "v_key_major", "free_committed_chunk"])
def test_cache_pins_catch_planted_mistakes(kind, monkeypatch):
    from test_oracle_cache import sequence_matches
    assert sequence_matches(seed=1, q_len=16, ring=256, window=100, prefill=150)
    ar, ap, P = _cache_mutant(kind)
    monkeypatch.setattr(oracle, "append_ring", ar)
    monkeypatch.setattr(oracle, "append_paged", ap)
    monkeypatch.setattr(oracle, "PagerModel", P)
    assert not sequence_matches(seed=1, q_len=16, ring=256, window=100, prefill=150)


# --- host paging and the resident subset: planted mistakes --------------------------------------

def _resident_mutant(kind):
    from oracle import cache as C

    def attention_resident(q, k_pool, v_pool, chunk_ids, slots, ctx_len, scale=None, dtype="bf16"):
        qf = A.to_f64(q, dtype)
        q_len, _, d = qf.shape
        pos, ks, ko = [], [], []
        for c, s in zip(chunk_ids, slots):
            base = s if kind == "slot_as_position" else c
            for t in range(C.CHUNK):
                if kind == "no_context_bound" or c * C.CHUNK + t < ctx_len:
                    pos.append(base * C.CHUNK + t)
                    ks.append(s)
                    ko.append(t)
        pos, ks, ko = np.array(pos), np.array(ks), np.array(ko)
        kp, vp = np.asarray(k_pool), np.asarray(v_pool)
        return A.attend_rows(qf, lambda g: A.to_f64(kp[ks, g, ko, :], dtype),
                             lambda g: A.to_f64(vp[ks, g, :, ko], dtype), pos,
                             ctx_len - q_len + np.arange(q_len), 0, 1.0 / math.sqrt(d),
                             kp.shape[1])
    return attention_resident


@pytest.mark.parametrize("kind", ["slot_as_position", "no_context_bound"])
def test_resident_pins_catch_planted_mistakes(kind, monkeypatch):
    from test_oracle_cache import test_resident_subset_matches_sdpa_with_mask as pin
    pin(1500, 16, (0, 3, 7, 8, 20, 21, 22, 23))
    monkeypatch.setattr(oracle, "attention_resident", _resident_mutant(kind))
    with pytest.raises(AssertionError):
        pin(1500, 16, (0, 3, 7, 8, 20, 21, 22, 23))


def test_page_out_without_v_is_caught(monkeypatch):
    from test_oracle_cache import test_page_out_in_round_trip_is_bit_exact as pin

    def page_out(k_pool, v_pool, slots, chunk_ids, k_host, v_host):
        kh, vh = np.array(k_host, copy=True), np.array(v_host, copy=True)
        for s, c in zip(slots, chunk_ids):
            kh[c] = k_pool[s]
        return kh, vh

    pin()
    monkeypatch.setattr(oracle, "page_out", page_out)
    with pytest.raises(AssertionError):
        pin()


def test_evicting_the_partial_tail_chunk_is_caught(monkeypatch):
    from test_oracle_cache import test_pager_model_evict_restore_policy_and_errors as pin
    from oracle import cache as C

    class Pager(C.PagerModel):
        def evict(self, chunk_ids):
            full = -(-self.ctx // C.CHUNK)             # ceil: the partly written chunk too
            ids = list(chunk_ids)
            if len(set(ids)) != len(ids) or any(not 0 <= c < full or self.table[c] < 0
                                                for c in ids):
                raise ValueError("evict")
            slots = [self.table[c] for c in ids]
            for c in ids:
                self.free.append(self.table[c])
                self.table[c] = C.PAGED_OUT
            return slots

    pin()
    monkeypatch.setattr(oracle, "PagerModel", Pager)
    with pytest.raises((AssertionError, pytest.fail.Exception)):   # "DID NOT RAISE"
        pin()


# --- the merge and the accept: planted mistakes in copies of lse_merge / greedy_accept ---------

def _merge_mutant(kind):
    def lse_merge(parts):
        lses = np.stack([np.asarray(l, dtype=np.float64) for _, l in parts])
        outs = np.stack([np.asarray(o, dtype=np.float64) for o, _ in parts])
        M = lses.max(axis=0)
        has = np.isfinite(M)
        Mz = np.where(has, M, 0.0) if kind != "no_max_shift" else np.zeros_like(M)
        w = np.where(np.isfinite(lses), np.exp(lses - Mz[None]), 0.0)
        if kind == "empty_part_weighted":
            w = np.where(np.isfinite(lses), w, 1.0)
        if kind == "equal_weights":
            w = np.where(np.isfinite(lses), 1.0, 0.0)
        tot = w.sum(axis=0)
        num = (w[..., None] * outs).sum(axis=0)
        out = np.zeros(outs.shape[1:], dtype=np.float64)
        out[has] = num[has] if kind == "no_normalise" else num[has] / tot[has][..., None]
        lse = np.full(M.shape, -np.inf)
        lse[has] = M[has] if kind == "lse_is_max" else M[has] + np.log(tot[has])
        return out, lse
    return lse_merge


def _merge_pins():
    import test_oracle_attention as T
    T.test_p9_split_merge_equals_unsplit(500)
    T.test_p9_merge_skips_empty_parts()
    T.test_p9_merge_at_logits_beyond_exp_range()


@pytest.mark.parametrize("kind", ["no_max_shift", "empty_part_weighted", "equal_weights",
                                  "no_normalise", "lse_is_max"])
def test_merge_pins_catch_planted_mistakes(kind, monkeypatch):
    _merge_pins()
    monkeypatch.setattr(oracle, "lse_merge", _merge_mutant(kind))
    with np.errstate(over="ignore", invalid="ignore"), pytest.raises(AssertionError):
        _merge_pins()


def _accept_mutant(kind):
    def greedy_accept(logits, proposals, scan=False):
        L = np.asarray(logits, dtype=np.float32)
        prop = np.asarray(proposals, dtype=np.int64)
        k = prop.shape[0]
        if kind == "last_maximum":                 # ties go to the higher index
            t = L.shape[1] - 1 - np.argmax(L[:, ::-1], axis=1)
        else:
            t = np.argmax(L, axis=1)
        if kind == "row_shift":                    # draft r checked against the row after it
            agree = [t[min(r + 1, k)] == prop[r] for r in range(k)]
        else:
            agree = [t[r] == prop[r] for r in range(k)]
        if kind == "count_agreements":             # agreements anywhere, not the prefix
            a = int(sum(agree))
        else:
            a = next((r for r in range(k) if not agree[r]), k)
        if kind == "no_target_token":
            committed = prop[:a]
        elif kind == "target_token_of_last_row":
            committed = np.concatenate([prop[:a], t[k:k + 1]])
        else:
            committed = np.concatenate([prop[:a], t[a:a + 1]])
        return a, committed.astype(np.int32), t.astype(np.int32)
    return greedy_accept


def _accept_pins():
    import test_oracle_accept as T
    for k in (0, 1, 2, 3):
        T.test_p10_brute_force_small_vocab_with_ties(k)
    T.test_signed_zero_tie_takes_lower_index()
    for a in (0, 7, 16):
        T.test_planted_prefix_is_recovered(a)
    T.test_exact_greedy_equivalence_on_a_toy_target()


@pytest.mark.parametrize("kind", ["last_maximum", "row_shift", "count_agreements",
                                  "no_target_token", "target_token_of_last_row"])
def test_accept_pins_catch_planted_mistakes(kind, monkeypatch):
    _accept_pins()
    monkeypatch.setattr(oracle, "greedy_accept", _accept_mutant(kind))
    with pytest.raises(AssertionError):
        _accept_pins()


def test_unmutated_accept_copy_passes_the_pins(monkeypatch):
    """The copy the mutants start from is itself correct (so each mutant differs by one mistake)."""
    monkeypatch.setattr(oracle, "greedy_accept", _accept_mutant("none"))
    _accept_pins()
    monkeypatch.setattr(oracle, "lse_merge", _merge_mutant("none"))
    _merge_pins()
