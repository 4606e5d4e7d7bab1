"""MI355X-native Kimi Delta Attention (KDA) forward operator.

The operator lives in libkda.so (HIP kernels for gfx950 behind the C ABI of
include/kda.h); `gated_delta_rule_10_amd.kda` is its Python binding and
`gated_delta_rule_10_amd.inputs` draws seeded synthetic inputs.
"""

__all__ = ["kda_chunk_fwd", "kda_decode_step", "kda_chunk_fwd_workspace_size", "kda_chunk_fwd_ex",
           "kda_decode_step_ex", "kda_chunk_fwd_ex_noalloc", "kda_abi_version", "kda_status_string", "KDAError"]


def __getattr__(name):
    # the binding imports torch; load it only when one of its names is used
    if name in __all__:
        from . import kda
        return getattr(kda, name)
    raise AttributeError(name)
