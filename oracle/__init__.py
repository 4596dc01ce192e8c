"""fp64 CPU oracle of the sparse-MoE block -- test infrastructure only.

Only the tests, the smoke check and the benchmark's CPU-baseline leg import
this package.  The HIP library never calls it and shares no code with it.
"""
from .moe_oracle import *  # noqa: F401,F403
from . import moe_oracle  # noqa: F401
