"""ctypes loader for the HIP library ``libattn.so`` (C ABI in include/attn.h).

There is no fallback: if the library is missing, ``load()`` raises.
"""

from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libattn.so")

# attn_status values (include/attn.h).
ATTN_OK = 0
ATTN_ERR_NULL_POINTER = -1
ATTN_ERR_BAD_SHAPE = -2
ATTN_ERR_GQA_RATIO = -3
ATTN_ERR_UNSUPPORTED_HDIM = -4
ATTN_ERR_UNSUPPORTED_DTYPE = -5
ATTN_ERR_BAD_SCALE = -6
ATTN_ERR_MISALIGNED = -7
ATTN_ERR_ALIASING = -8
ATTN_ERR_NO_DEVICE = -9
ATTN_ERR_LAUNCH = -10
ATTN_ERR_WORKSPACE = -11
ATTN_ERR_BAD_ARGUMENT = -12
ATTN_ERR_SCRATCH_LIMIT = -13

# attn_decode_noalloc's scratch array, per GPU (include/attn.h)
ATTN_DECODE_SCRATCH_BYTES = 8 << 20

# attn_dtype values.
ATTN_DTYPE_F16 = 0
ATTN_DTYPE_BF16 = 1

_lib = None


def load() -> ctypes.CDLL:
    """Load the library once and declare the exported signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"HIP library {LIB_PATH} is not built; run `python -m exact_tiled_attention_35_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, ci, cf = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.attn_fwd.argtypes = [vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, cf, ci, ci, vp]
    lib.attn_fwd.restype = ci
    lib.attn_fwd_ext.argtypes = [vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, cf, ci, ci, ci, vp, cf,
                                 ci, vp]
    lib.attn_fwd_ext.restype = ci
    lib.attn_fwd_varlen.argtypes = [vp] * 7 + [ci] * 7 + [cf, ci, ci, vp]
    lib.attn_fwd_varlen.restype = ci
    lib.attn_fwd_blocksparse.argtypes = [vp] * 6 + [ci] * 7 + [cf, ci, ci, vp]
    lib.attn_fwd_blocksparse.restype = ci
    lib.attn_bwd.argtypes = [vp] * 10 + [ci, ci, ci, ci, ci, ci, cf, ci, ci, vp]
    lib.attn_bwd.restype = ci
    lib.attn_bwd_blocksparse.argtypes = [vp] * 11 + [ci] * 7 + [cf, ci, ci, vp]
    lib.attn_bwd_blocksparse.restype = ci
    lib.attn_bwd_varlen.argtypes = [vp] * 12 + [ci] * 8 + [cf, ci, ci, vp]
    lib.attn_bwd_varlen.restype = ci
    lib.attn_bwd_ext.argtypes = [vp] * 10 + [ci] * 6 + [cf, ci, ci, ci, vp, cf, ci, vp]
    lib.attn_bwd_ext.restype = ci
    lib.attn_decode.argtypes = [vp] * 9 + [ctypes.c_size_t] + [ci] * 7 + [cf, ci, ci, ci, vp]
    lib.attn_decode.restype = ci
    lib.attn_decode_noalloc.argtypes = [vp] * 8 + [ci] * 7 + [cf, ci, ci, ci, vp]
    lib.attn_decode_noalloc.restype = ci
    lib.attn_decode_num_splits.argtypes = [ci] * 6
    lib.attn_decode_num_splits.restype = ci
    lib.attn_decode_workspace_size.argtypes = [ci] * 5
    lib.attn_decode_workspace_size.restype = ctypes.c_size_t
    lib.attn_status_string.argtypes = [ci]
    lib.attn_status_string.restype = ctypes.c_char_p
    lib.attn_version.argtypes = []
    lib.attn_version.restype = ctypes.c_char_p
    _lib = lib
    return lib
