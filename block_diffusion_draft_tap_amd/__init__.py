"""MI355X (gfx950) hot path of the DFlash KV-injection block drafter.

The compute lives in libdflash.so (HIP kernels behind a C ABI, include/dflash.h);
`binding` is its thin Python binding.
"""

from . import binding  # noqa: F401
from .binding import (DeviceModel, KVCache, Weight, workspace, lm_head_workspace, verify_workspace,  # noqa: F401
                      dflash_query, dflash_context_project, dflash_ctx_kv_append, dflash_draft_layer,
                      dflash_draft_forward, dflash_lm_head_argmax, dflash_verify_greedy, dflash_invocations,
                      check, DflashError)
