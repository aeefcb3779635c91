"""Blockwise exact ring attention for one MI355X (gfx950).

The compute path is a C-ABI shared library of hand-written HIP kernels
(``libra_attn.so``, built from ``csrc/``); this package only marshals
arguments to it.  Importing the package does not load the library; the
first call does, and raises if the library is missing -- there is no CPU
fallback.
"""
from .api import (  # noqa: F401
    RAError,
    blockwise_attn_fwd,
    blockwise_attn_bwd,
    blockwise_attn_bwd_preprocess,
    blockwise_attn_bwd_dkdv,
    blockwise_attn_bwd_dq,
    blockwise_attn_fwd_step,
    blockwise_attn_fwd_finalize,
    attn_merge,
    blockwise_attn_bwd_step,
    blockwise_attn_bwd_dbias_reduce,
    blockwise_attn_bwd_dbias,
    blockwise_attn_bwd_noalloc,
    blockwise_ffn_fwd,
    blockwise_ffn_bwd,
    blockwise_attn_bwd_finalize,
    bwd_workspace_size,
    library_path,
    load_library,
)
