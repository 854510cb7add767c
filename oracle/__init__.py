"""CPU oracle for the routed-expert MoE FFN path (test infrastructure only).

Plain, slow, obviously-correct NumPy code that the parity tests, the
round-trip smoke check and the bench's CPU-baseline leg compare the HIP
library against.  Nothing on the product path imports it, and it imports
nothing from the product package or its sources.
"""
from .ref import *  # noqa: F401,F403
