"""CPU oracle for the HSTU jagged pointwise-attention path (test infrastructure only).

Only tests, the package smoke check and the benchmark's CPU-baseline leg may use it.
"""
from .hstu_oracle import *  # noqa: F401,F403
