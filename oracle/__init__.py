"""CPU oracle (float64 numpy) of the EDiT layer and the MM-EDiT hybrid.

Test infrastructure only: imported by tests, the smoke check and the
benchmark's CPU-baseline leg, never by the HIP library or its binding.
"""
from .edit_oracle import *  # noqa: F401,F403
from . import edit_oracle  # noqa: F401
