"""Longformer sparse self-attention (forward and backward) for AMD Instinct MI355X (gfx950).

The compute lives in liblfattn.so (C ABI, include/lf_attn.h); this package
only marshals torch tensors into it.
"""
from .binding import (LF_BF16, LF_E_HIP, LF_E_INVALID, LF_E_NOMEM, LF_E_UNSUPPORTED, LF_F32, Prepared,
                      LF_OK, LIB_PATH, LfError, attn_bwd, attn_fwd, attn_fwd_global_rows, last_error, load, raw_bwd,
                      raw_fwd)

__all__ = ["attn_fwd", "attn_fwd_global_rows", "attn_bwd", "raw_bwd", "Prepared", "load", "raw_fwd", "last_error", "LfError", "LIB_PATH", "LF_F32", "LF_BF16",
           "LF_OK", "LF_E_INVALID", "LF_E_UNSUPPORTED", "LF_E_NOMEM", "LF_E_HIP"]
