"""CPU oracle for the DFlash block drafter.

TEST INFRASTRUCTURE ONLY: imported by the tests, the package smoke check and
the benchmark's CPU-baseline leg, never by the library's product path.
"""

from . import dflash_oracle
from .dflash_oracle import *  # noqa: F401,F403
