"""Plain CPU oracle of the TriAttention eviction pass.

TEST INFRASTRUCTURE ONLY: imported by the tests, by the package smoke check
and by the benchmark's CPU-baseline leg, never by the product path.
"""
from .oracle import *  # noqa: F401,F403
