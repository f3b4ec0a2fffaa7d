"""CPU oracle of the MoE layer (fp64, numpy).  Test infrastructure: only the
tests, the smoke check and the benchmark's CPU-baseline leg use it."""
from .moe_oracle import *  # noqa: F401,F403
