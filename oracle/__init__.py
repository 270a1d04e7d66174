"""CPU oracle of the GPTQ layer quantizer (float64).

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check and by the
benchmark's CPU-baseline leg; never by the product path.
"""
from .gptq_oracle import *  # noqa: F401,F403
from .gptq_oracle import __all__  # noqa: F401
