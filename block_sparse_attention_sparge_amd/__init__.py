"""MI355X-native (gfx950) SpargeAttn-style block-sparse attention forward.

The compute lives in a C-ABI shared library of hand-written HIP kernels
(``libsparge.so``, declared in ``include/sparge.h``).  The Python layer only
marshals torch tensors into that ABI; it is loaded on first use, and every
entry point raises if the library cannot be loaded -- there is no fallback.
"""
from .ops import (  # noqa: F401
    SpargeError, attn_combine, build_block_map, dense_fmha_fwd, load_library,
    sparse_fmha_fwd, block_map_workspace_bytes, validate_lut,
)

__all__ = [
    "SpargeError", "attn_combine", "build_block_map", "dense_fmha_fwd",
    "load_library", "sparse_fmha_fwd", "block_map_workspace_bytes", "validate_lut",
]
