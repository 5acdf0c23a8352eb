"""CPU oracle of the LiftQuant decode operator and the reference sign packer.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product path (``bit_matmul_amd``).
It shares no code with the HIP library.
"""
from . import liftquant_ref, refpack

__all__ = ["liftquant_ref", "refpack"]
