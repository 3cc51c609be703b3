"""fp64 CPU oracle for CoWindow Attention (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg import
this package; the GPU library never does.
"""
from .cowa_oracle import *  # noqa: F401,F403
from .cowa_oracle import Pattern, MODE_COWA, MODE_CAUSAL  # noqa: F401
