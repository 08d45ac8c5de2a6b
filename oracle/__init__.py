"""fp64 CPU oracle of the routed low-bit MoE FFN layer.

TEST INFRASTRUCTURE: imported only by the tests, the smoke check and the
benchmark's CPU-baseline leg.  It shares no code with the HIP library.
"""
from .moe_oracle import *  # noqa: F401,F403
from . import moe_oracle  # noqa: F401
