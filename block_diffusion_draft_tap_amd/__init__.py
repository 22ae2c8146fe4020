"""MI355X (gfx950) hot path of the DFlash KV-injection block drafter.

The compute lives in libdflash.so (HIP kernels behind a C ABI, include/dflash.h);
`binding` is its thin Python binding. The library is loaded on first use of
any binding name (so `block_diffusion_draft_tap_amd.build` can run before it
exists); a missing library raises ImportError there.
"""

_BINDING_NAMES = (
    "DeviceModel", "KVCache", "Weight", "workspace", "lm_head_workspace", "verify_workspace", "kv_prefill_workspace",
    "dflash_query", "dflash_context_project", "dflash_ctx_kv_append", "dflash_draft_layer",
    "dflash_draft_forward", "dflash_lm_head_argmax", "dflash_verify_greedy", "dflash_invocations",
    "dflash_trace_begin", "dflash_trace_end", "DsparkHead", "dspark_workspace",
    "dflash_draft_forward_dspark", "dflash_verify_greedy_lengths", "dflash_draft_round", "round_workspace",
    "dflash_verify_from_hidden", "verify_hidden_workspace", "int4_prefill_workspace",
    "check", "DflashError",
)


def __getattr__(name):
    if name == "binding" or name in _BINDING_NAMES:
        import importlib

        binding = importlib.import_module(".binding", __name__)
        return binding if name == "binding" else getattr(binding, name)
    raise AttributeError(name)
