"""CPU oracle of the token-choice MoE FFN forward pass (float64, NumPy).

TEST INFRASTRUCTURE.  Only the test-suite, the smoke check of the package
entry file and the CPU-baseline leg of the benchmark may import this package.
The HIP library never calls it and it never calls the HIP library; the two
share no code.  See ``moe_ref`` for the definitions and their sources.
"""
from .moe_ref import *  # noqa: F401,F403
