"""fp64 CPU oracle for ring attention (one rank's share).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
bench's CPU-baseline leg, never by the product path.  It shares no code with
the HIP library.
"""
from .ring_oracle import *  # noqa: F401,F403
