"""Exact tiled attention forward for AMD MI355X (gfx950).

The computation runs in hand-written HIP kernels behind a C ABI
(``include/attn.h``, built into ``libattn_fwd.so``); this package is the thin
Python binding over it.
"""

from .attention import AttnError, attn_fwd, attn_fwd_ptr, attn_status_string, attn_version  # noqa: F401

__version__ = "0.1.0"
