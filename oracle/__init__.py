"""CPU oracle for the fused producer/consumer gather-GEMM.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import this package:
only the tests, the smoke check and the benchmark's CPU-baseline leg use it.
It shares no code with the HIP library and never calls it.
"""
from .fg_oracle import *  # noqa: F401,F403
