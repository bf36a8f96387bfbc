"""fp64 CPU oracle of the expert-cached MoE layer.  TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The product path (the HIP library and its binding) never calls
it and shares no code with it.
"""
from .moe_oracle import *  # noqa: F401,F403
