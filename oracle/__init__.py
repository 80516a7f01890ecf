"""fp64 CPU oracle for the speculative-decoding verify step.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it.  The product (``ring_kv_amd``
and its HIP library) never imports, links or calls anything here, and this
package never imports the product: the two share no code.

What it computes, and where the method is stated:

* ``attention``: the verify block's attention as the plain softmax definition,
  two passes per row in float64, over the three KV stores: contiguous rows,
  the sliding-window position ring, and the paged pool of 64-token chunks
  (lucebox post "Laguna XS 2.1 33B on a RTX 3090: 296 tok/s peak, 152 tok/s at
  256K context": "Three optimizations" item 1 for the 64-token chunk pool, item 3
  "Ring caches for the sliding-window layers" for slot = pos mod 2048 and the
  512-token window; "The model, fast MoE with a drafter in the box" for the one
  batched forward over the 16 proposals).
* ``merge``: the log-sum-exp merge of attention partials over disjoint key sets
  (a split of the key range; exact up to rounding).
* ``accept``: greedy acceptance, committing the longest drafted prefix on which
  the target's argmax agrees plus the target's next token (same post, "TL;DR" and
  "The model, fast MoE with a drafter in the box": exact greedy equivalence).
* ``cache``: appending the verify block's own K/V rows to the ring and the pool
  before its attention, and committing the accepted ones (slot = pos mod 2048; a
  pool chunk gets a slot when first written and gives it back if the block's rows
  in it are all rejected), with ``PagerModel``, the slot bookkeeping; paging whole chunks
  out to a host chunk store and back in, and attention over the resident subset of the
  pool (same post, "Three optimizations", item 1).

Parity pins: every function here is pinned in ``tests/test_oracle_*.py`` by
closed forms, invariants, brute force or a library routine; none is "parity
unpinned".
"""
from .attention import (attend_rows, attention_contiguous, attention_paged,  # noqa: F401
                        attention_ring, bf16_to_f64, gather_paged, gather_ring,
                        key_bounds, to_f64)
from .merge import attention_partial, lse_merge  # noqa: F401
from .accept import first_argmax, greedy_accept  # noqa: F401
from .cache import (PAGED_OUT, PagerModel, append_paged, append_ring,  # noqa: F401
                    attention_resident, page_in, page_out)
