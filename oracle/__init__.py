"""fp64 CPU oracle for the IndexCache / DSA hot path.

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
benchmark's cpu_baseline leg, never by the product path.
"""
from .dsa_oracle import *  # noqa: F401,F403
