"""CPU oracle of the DFlash drafter hot path (numpy, fp64).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
bench's CPU-baseline leg. The GPU library never imports or calls it.
"""
from .dflash_oracle import *  # noqa: F401,F403
from .dflash_oracle import DraftCache  # noqa: F401
