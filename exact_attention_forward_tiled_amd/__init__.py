"""MI355X-native (gfx950) fused, tiled, exact attention forward.

The compute path is libattn.so (hand-written HIP kernels behind the C ABI in
include/attn.h); this package is its thin Python binding.  The binding is
imported on first use of any of its names, so that the build module can run
before the library exists; using a name when libattn.so is missing raises
ImportError (there is no fallback path).
"""

import importlib

_BINDING_NAMES = ("AttnError", "EXPORTS", "attn_bwd", "attn_bwd_ex", "attn_bwd_noalloc", "attn_fwd",
                  "attn_fwd_ex",
                  "attn_fwd_mxfp4", "attn_fwd_mxfp4_ex", "attn_fwd_mxfp8", "attn_fwd_mxfp8_ex",
                  "attn_quantize_mxfp4_cols_t", "attn_quantize_mxfp4_rows",
                  "attn_quantize_mxfp8_cols_t", "attn_quantize_mxfp8_rows", "bwd", "check",
                  "fwd", "fwd_mxfp4", "fwd_mxfp8", "make_opts", "quantize_mxfp4_cols_t",
                  "quantize_mxfp4_rows", "quantize_mxfp8_cols_t", "quantize_mxfp8_rows",
                  "STATS_COUNTERS", "lib")

__all__ = list(_BINDING_NAMES)


def __getattr__(name):
    if name in _BINDING_NAMES:
        binding = importlib.import_module(".binding", __name__)
        return getattr(binding, name)
    raise AttributeError(f"module {__name__!r} has no attribute {name!r}")
