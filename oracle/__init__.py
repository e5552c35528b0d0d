"""fp64 CPU oracle of the MoE layer. Test infrastructure only: imported by the tests, the smoke
check and the benchmark's CPU-baseline leg, never by the library."""
from .moe_oracle import *  # noqa: F401,F403
