"""Pins of the greedy-accept oracle: brute force, construction, and exact greedy
equivalence on a toy target model (CPU only)."""
import itertools

import numpy as np
import pytest

import oracle
from synth import accept_case


def _literal(logits, prop):
    """Longest agreeing prefix by a literal loop over Python lists."""
    rows = [list(map(float, r)) for r in np.asarray(logits, np.float32)]
    t = [r.index(max(r)) for r in rows]            # list.index: the first maximum
    a = 0
    while a < len(prop) and prop[a] == t[a]:
        a += 1
    return a, list(prop[:a]) + [t[a]], t


@pytest.mark.parametrize("k", [0, 1, 2, 3])
def test_p10_brute_force_small_vocab_with_ties(k):
    V = 3
    g = np.random.default_rng(100 + k)
    for trial in range(20):
        # values from {0, 1, 2} so that ties are common
        L = g.integers(0, 3, size=(k + 1, V)).astype(np.float32)
        for prop in itertools.product(range(V), repeat=k):
            a, com, t = oracle.greedy_accept(L, np.array(prop, np.int32))
            la, lcom, lt = _literal(L, prop)
            assert a == la and list(com) == lcom and list(t) == lt
            a2, com2, t2 = oracle.greedy_accept(L, np.array(prop, np.int32), scan=True)
            assert a2 == a and list(com2) == list(com) and list(t2) == list(t)


def test_signed_zero_tie_takes_lower_index():
    L = np.array([[-0.0, 0.0, -1.0], [0.0, -0.0, -5.0]], np.float32)
    a, com, t = oracle.greedy_accept(L, np.array([0], np.int32))
    assert list(t) == [0, 0] and a == 1 and list(com) == [0, 0]
    assert oracle.first_argmax(L[0]) == 0


@pytest.mark.parametrize("accept", [0, 1, 7, 15, 16])
def test_planted_prefix_is_recovered(accept):
    c = accept_case(5, accept, 16, 4096, 0.0, accept=accept)
    a, com, t = oracle.greedy_accept(c.logits, c.proposals)
    assert a == accept == c.planted_accept
    np.testing.assert_array_equal(t, c.planted_targets)
    np.testing.assert_array_equal(com, np.concatenate([c.proposals[:a], c.planted_targets[a:a + 1]]))
    assert len(com) == a + 1


@pytest.mark.parametrize("vocab", [1, 2, 4095, 4097])
def test_vocab_edges(vocab):
    c = accept_case(6, vocab, 16, vocab, 1e-3, "uniform")
    a, com, t = oracle.greedy_accept(c.logits, c.proposals)
    assert a == c.planted_accept
    np.testing.assert_array_equal(t, c.planted_targets)
    if vocab == 1:
        assert a == 16 and list(com) == [0] * 17


def test_planted_margin_holds():
    c = accept_case(7, 0, 16, 65536, 1e-3, "binomial")
    for r in range(17):
        row = np.sort(c.logits[r])
        assert np.float32(row[-1] - row[-2]) >= np.float32(1e-3)
    c0 = accept_case(8, 0, 16, 4096, 0.0, "uniform")
    for r in range(17):
        row = np.sort(c0.logits[r])
        assert row[-1] > row[-2]                     # unique, by as little as one ulp


def test_exact_greedy_equivalence_on_a_toy_target():
    """Speculative decoding with this accept rule emits exactly the greedy sequence.

    Toy target: next-token logits are a fixed random function of the last two tokens.
    Drafts are partly right (copied from a greedy run) and partly random."""
    V, k, n_out = 11, 4, 60
    table = np.random.default_rng(9).standard_normal((V, V, V)).astype(np.float32)

    def logits_after(seq):
        return table[seq[-2], seq[-1]]

    greedy = [3, 5]
    while len(greedy) < 2 + n_out:
        greedy.append(int(np.argmax(logits_after(greedy))))

    g = np.random.default_rng(10)
    seq = [3, 5]
    steps = 0
    while len(seq) < 2 + n_out:
        pos = len(seq)
        prop = [greedy[pos + r] if (pos + r < len(greedy) and g.random() < 0.7)
                else int(g.integers(0, V)) for r in range(k)]
        rows = [logits_after(seq + prop[:r]) for r in range(k + 1)]
        a, com, _ = oracle.greedy_accept(np.stack(rows), np.array(prop, np.int32))
        seq.extend(int(x) for x in com)
        steps += 1
    assert seq[:2 + n_out] == greedy[:2 + n_out]
    assert steps < n_out        # more than one token per step on average
