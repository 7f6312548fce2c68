"""CPU oracle for the per-GPU MoE expert layer (test infrastructure only).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package; the product path never does.
"""
from .moe_oracle import *  # noqa: F401,F403
from . import moe_oracle  # noqa: F401
