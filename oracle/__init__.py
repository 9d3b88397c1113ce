"""CPU fp64 oracle for paged attention decode.

TEST INFRASTRUCTURE: only tests/, the smoke check and the benchmark's CPU
baseline leg may import this package. The GPU library never calls it.
Every function here is pinned by tests against closed forms, brute force and
a library routine; none is marked "parity unpinned".
"""
from .tolerance import bf16_step, compare, rounding_allowance
from .append import append_rows, new_token_slots
from . import gqla, fp8
from .attention import (PAGE, attend_bruteforce, attend_online, attend_two_pass,
                        bf16_to_f64, combine, gather_pages, scale_as_received,
                        softmax_weights, value_spread, visible_keys)

__all__ = ["gqla", "fp8", "compare", "bf16_step", "rounding_allowance", "append_rows", "new_token_slots", "PAGE", "attend_bruteforce", "attend_online", "attend_two_pass",
           "bf16_to_f64", "combine", "gather_pages", "scale_as_received",
           "softmax_weights", "value_spread", "visible_keys"]
