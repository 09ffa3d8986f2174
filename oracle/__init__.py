"""CPU oracle for the NF4 + Double-Quantisation QLoRA linear layer.

Test infrastructure only: imported by the tests, the package smoke check and
the benchmark's CPU-baseline leg, never by the product path.
"""
from .nf4_oracle import *  # noqa: F401,F403
from .nf4_oracle import BLOCK, DQ_GROUP, INT8_STEP  # noqa: F401
