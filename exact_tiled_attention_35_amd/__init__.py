"""Exact tiled attention (forward and backward) for AMD MI355X (gfx950).

The computation runs in hand-written HIP kernels behind a C ABI
(``include/attn.h``, built into ``libattn.so``); this package is the thin
Python binding over it.
"""

from .attention import (  # noqa: F401
    AttnError,
    attention,
    attn_bwd,
    attn_bwd_blocksparse,
    attn_bwd_blocksparse_ptr,
    attn_bwd_ext_ptr,
    attn_bwd_ptr,
    attn_bwd_varlen,
    attn_bwd_varlen_ptr,
    attn_decode,
    attn_decode_noalloc,
    attn_decode_noalloc_ptr,
    attn_decode_num_splits,
    attn_decode_ptr,
    attn_decode_workspace_size,
    BLOCK_MASK_SIZE,
    attn_fwd,
    attn_fwd_blocksparse,
    attn_fwd_blocksparse_ptr,
    attn_fwd_ext_ptr,
    attn_fwd_ptr,
    attn_fwd_varlen,
    attn_fwd_varlen_ptr,
    attn_status_string,
    attn_version,
)

__version__ = "0.3.0"
