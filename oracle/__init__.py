"""fp64 CPU oracle of the routed MoE decode step -- test infrastructure only.

Only the tests, the smoke check and the benchmark's CPU-baseline leg import
this package; the product path never does.  See moe_oracle.py.
"""
from .moe_oracle import *  # noqa: F401,F403
from .moe_oracle import bf16_to_f64, silu  # noqa: F401
from . import reader_oracle as reader  # noqa: F401  (the channel-selection reader)
