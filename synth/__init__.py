"""Seeded synthetic inputs for the verify-step attention and the greedy accept.

This package is shared by the tests, the bench and the smoke check. It holds
none of the method's arithmetic: only random draws, the bf16 rounding of those
draws, the scatter of contiguous K/V rows into the chunked store layouts that
``include/ring_kv.h`` defines, and the planting of known answers (a chosen
argmax per logit row, a chosen agreement prefix).
"""
from .inputs import *  # noqa: F401,F403
from .workloads import *  # noqa: F401,F403
