"""CPU oracle of the fp8 block-quantized MoE expert layer.

TEST INFRASTRUCTURE ONLY: imported by tests, by the smoke check and by the
benchmark's CPU-baseline leg, never by the product path.  It shares no code
with the HIP library.
"""
from .moe_oracle import *  # noqa: F401,F403
