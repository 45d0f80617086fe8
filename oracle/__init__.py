"""Plain fp64 CPU oracle for exact attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import, call or execute anything in this package.  The HIP
library never imports it, and the oracle imports nothing from the HIP side:
the two share no kernels, headers, helpers, tables or pre/post-processing.

What it computes follows the pages' statement of exact attention
(tokenwerk.de "FlashAttention", section "Was FlashAttention veraendert";
hysenlabs.com "FlashAttention: exakte Attention-Kernel fuer CUDA und ROCm",
section "Die Schnittstellen von flash_attn_func bis KV-Cache"):
``out = softmax(Q @ K^T * softmax_scale) @ V`` with the full score matrix
written out, per (batch, query head).
"""

from .exact import (  # noqa: F401
    attention,
    attention_backward,
    attention_varlen,
    attention_backward_varlen,
    attention_block_sparse,
    attention_block_sparse_rows,
    attention_rows,
    kv_head_of,
    allowed_keys,
    materialised_score_bytes,
    visible_range,
)
