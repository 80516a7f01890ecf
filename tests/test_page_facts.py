"""The workload shapes and the oracle's window/ring rules against figures the lucebox
post prints (fixtures in tests/golden/page_facts.json, each with its section)."""
import json
import os

import numpy as np

import oracle
from synth import CHUNK, STACK_LAYERS, stack_layer_kind, workload

FACTS = {f["id"]: f for f in json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                                         "page_facts.json")))["facts"]}


def test_ring_slot_example():
    f = FACTS["ring_slot_rule"]
    c, _ = workload("ring_w512_r2048")
    assert c.ring_size == f["ring_size"] and c.pos0 == f["example_pos"]
    assert c.ring_head == f["example_slot"] == f["example_pos"] % f["ring_size"]


def test_masked_share_of_a_16k_span():
    f = FACTS["masked_share"]
    span = f["span_upper"]
    lo, hi = oracle.key_bounds(span - 1, f["window"])
    visible = hi - lo + 1
    assert visible == f["window"]
    assert round(100 * (1 - visible / span)) == f["masked_percent_rounded"]


def test_layer_pattern_and_block():
    f = FACTS["layer_pattern"]
    kinds = [stack_layer_kind(l) for l in range(STACK_LAYERS)]
    assert STACK_LAYERS == f["layers"] and kinds.count("ring") == f["window_layers"]
    b = FACTS["block"]
    c, _ = workload("paged_8k")
    assert c.q_len == b["proposals"] and c.n_q_heads * c.head_dim == b["hidden"]
    assert CHUNK == FACTS["chunk"]["chunk"] == c.chunk


def test_kv_sizes_consistent_with_the_post():
    c, _ = workload("paged_8k")
    per_pos = 2 * c.n_kv_heads * c.head_dim * 2          # K and V, bf16
    full = STACK_LAYERS * FACTS["full_kv_256k"]["context"] * per_pos
    assert abs(full / 2 ** 30 - FACTS["full_kv_256k"]["approx_gib"]) < 0.5
    freed = FACTS["layer_pattern"]["window_layers"] * (FACTS["masked_share"]["span_upper"] - 2048) * per_pos
    assert round(freed / 1e9) == FACTS["ring_vram_freed"]["approx_gb"]
    assert c.attended_positions() == 8192 and np.isclose(c.kv_bytes, 2 * 8192 * 1024)
