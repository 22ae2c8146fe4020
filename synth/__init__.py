"""Seeded synthetic workloads for the DFlash block drafter (inputs only)."""

from .configs import (Dims, CONFIGS, TINY, DEFAULT, WIDE, WIDE4, BATCHED, DFLASH2, GROUP, scaled,
                      WDTYPE_F32, WDTYPE_BF16, WDTYPE_INT4G64, ACT_GELU_TANH, ACT_SILU)
from . import gen
