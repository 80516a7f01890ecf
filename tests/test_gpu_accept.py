"""GPU greedy accept (HIP kernels through the C interface): bit-exact against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import ring_kv_amd as rk
from synth import accept_case, workload
from gpu_util import dev, say

pytestmark = pytest.mark.gpu


def _run(logits, prop):
    a, com, t = rk.verify_accept(dev(np.ascontiguousarray(logits, np.float32)),
                                 dev(np.ascontiguousarray(prop, np.int32)))
    torch.cuda.synchronize()
    return int(a.cpu()[0]), com.cpu().numpy(), t.cpu().numpy()


def _check(logits, prop, what):
    a, com, t = _run(logits, prop)
    ra, rcom, rt = oracle.greedy_accept(logits, prop)
    assert a == ra, f"{what}: accept {a} != {ra}"
    np.testing.assert_array_equal(t, rt)
    np.testing.assert_array_equal(com[:a + 1], rcom)
    assert np.all(com[a + 1:] == -1)
    return a


def test_named_workloads():
    _, acc = workload("contig_1k_f32")
    say("accept contig_1k_f32 [17 x 4096]")
    assert _check(acc.logits, acc.proposals, "c1") == acc.planted_accept
    _, acc = workload("stack_40l_131k", 0)
    say("accept stack [17 x 65536]")
    assert _check(acc.logits, acc.proposals, "c5") == acc.planted_accept


@pytest.mark.parametrize("accept", [0, 1, 9, 15, 16])
def test_planted_prefixes(accept):
    c = accept_case(20, accept, 16, 65536, 1e-3, accept=accept)
    say(f"accept planted a={accept}")
    assert _check(c.logits, c.proposals, f"a={accept}") == accept


@pytest.mark.parametrize("n_draft,vocab", [(16, 1), (16, 2), (16, 4095), (16, 4097), (0, 5000),
                                           (1, 3), (255, 1000), (16, 151936), (7, 65537)])
def test_sizes(n_draft, vocab):
    c = accept_case(21, vocab, n_draft, vocab, 0.0, "uniform")
    say(f"accept n_draft={n_draft} vocab={vocab}")
    assert _check(c.logits, c.proposals, f"{n_draft}x{vocab}") == c.planted_accept


def test_ties_take_the_lowest_index():
    g = np.random.default_rng(22)
    for trial in range(30):
        vocab = int(g.integers(2, 9000))
        L = g.integers(-3, 3, size=(17, vocab)).astype(np.float32)   # many exact ties
        if trial % 3 == 0:
            L[:, ::7] = np.float32(-0.0)
            L[:, 1::7] = np.float32(0.0)
        t = np.argmax(L, axis=1)
        a = int(g.integers(0, 17))
        prop = g.integers(0, vocab, size=16).astype(np.int32)
        prop[:a] = t[:a]
        say(f"accept ties trial {trial} vocab={vocab}")
        _check(L, prop, f"ties {trial}")


def test_random_rows_against_the_oracle():
    g = np.random.default_rng(23)
    for trial in range(20):
        vocab = int(g.integers(1000, 70000))
        L = g.standard_normal((17, vocab)).astype(np.float32)
        prop = np.argmax(L, axis=1)[:16].astype(np.int32)
        prop[int(g.integers(0, 16))] = int(g.integers(0, vocab))
        _check(L, prop, f"random {trial}")


@pytest.mark.parametrize("vocab", [262145, 300001, 1000003])
def test_more_than_64_parts(vocab):
    """Vocabularies above 64 parts of 4,096 logits, where each lane of a row's group also walks
    the parts past the first 64: maxima planted on both sides of part 64 and at the ragged end,
    and exact ties across it (the lower index wins)."""
    g = np.random.default_rng(24)
    L = g.standard_normal((17, vocab)).astype(np.float32)
    spots = [0, 4095, 4096, 262143, 262144, vocab - 2, vocab - 1]
    for r in range(17):
        L[r, spots[r % len(spots)]] = np.float32(9.0)
    L[7, [262144, vocab - 1]] = np.float32(11.0)        # tie past part 64: the lower wins
    L[8, [5, vocab - 1]] = np.float32(11.0)             # tie across part 64
    L[9, [262143, 262144]] = np.float32(11.0)           # tie straddling the part-64 boundary
    prop = np.argmax(L, axis=1)[:16].astype(np.int32)
    prop[12] = (prop[12] + 1) % vocab                   # disagreement at 12
    say(f"accept more than 64 parts vocab={vocab}")
    assert _check(L, prop, f"parts>64 {vocab}") == 12


def test_many_rows_many_parts():
    """255 drafts (256 rows, the most one call takes) at 38 parts per row: sixteen rounds of the
    final reduction's row groups."""
    g = np.random.default_rng(25)
    vocab = 151936
    L = g.standard_normal((256, vocab)).astype(np.float32)
    t = np.argmax(L, axis=1)
    prop = t[:255].astype(np.int32).copy()
    prop[200] = (prop[200] + 3) % vocab
    say("accept 256 rows x 151936")
    assert _check(L, prop, "256x151936") == 200
