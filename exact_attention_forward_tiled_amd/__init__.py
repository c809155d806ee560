"""MI355X-native (gfx950) fused, tiled, exact attention forward.

The compute path is libattn.so (hand-written HIP kernels behind the C ABI in
include/attn.h); this package is its thin Python binding.
"""

from .binding import (AttnError, EXPORTS, attn_fwd, attn_fwd_ex, attn_fwd_mxfp4,
                      attn_fwd_mxfp4_ex, attn_quantize_mxfp4_cols_t, attn_quantize_mxfp4_rows,
                      check, fwd, fwd_mxfp4, make_opts, quantize_mxfp4_cols_t,
                      quantize_mxfp4_rows)

__all__ = ["AttnError", "EXPORTS", "attn_fwd", "attn_fwd_ex", "attn_fwd_mxfp4",
           "attn_fwd_mxfp4_ex", "attn_quantize_mxfp4_rows", "attn_quantize_mxfp4_cols_t",
           "check", "fwd", "fwd_mxfp4", "make_opts", "quantize_mxfp4_rows",
           "quantize_mxfp4_cols_t"]
