"""CPU oracle of the P-EAGLE drafter hot path.

TEST INFRASTRUCTURE: only tests/, the smoke check and the benchmark's CPU
baseline may import this package.  The HIP library never calls it.
"""
from .peagle_oracle import *  # noqa: F401,F403
from . import peagle_oracle as po  # noqa: F401
