"""Python binding of the C ABI: argument marshalling only.

``attn_fwd`` and ``attn_bwd`` check that the torch tensors match the C
ABI's layout contract, allocate the outputs with torch (device memory is
torch's job), and call the library's entry points of the same names on
torch's current HIP stream.  Every step of the computation runs in the HIP
kernels.  ``attention`` wraps the two as a torch autograd function.
"""

from __future__ import annotations

import math

import torch

from . import _lib

_DTYPE_CODE = {torch.float16: _lib.ATTN_DTYPE_F16, torch.bfloat16: _lib.ATTN_DTYPE_BF16}


class AttnError(RuntimeError):
    """A nonzero attn_status from the library; ``.code`` holds the value."""

    def __init__(self, code: int):
        self.code = code
        super().__init__(attn_status_string(code))


def attn_status_string(status: int) -> str:
    return _lib.load().attn_status_string(int(status)).decode()


def attn_version() -> str:
    return _lib.load().attn_version().decode()


def attn_fwd_ptr(q: int, k: int, v: int, out: int, lse: int, B: int, Hq: int, Hkv: int,
                 Nq: int, Nk: int, d: int, scale: float, causal: bool, dtype: int,
                 stream: int = 0) -> int:
    """The C entry point with raw integer pointers; returns the attn_status."""
    return _lib.load().attn_fwd(q, k, v, out, lse, int(B), int(Hq), int(Hkv), int(Nq), int(Nk),
                                int(d), float(scale), int(bool(causal)), int(dtype), stream or None)


def _check_qkv(q, k, v):
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-D [B, N, H, d]")
    B, Nq, Hq, d = q.shape
    Bk, Nk, Hkv, dk = k.shape
    if tuple(v.shape) != tuple(k.shape) or Bk != B or dk != d:
        raise ValueError(f"shape mismatch: q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    if q.dtype not in _DTYPE_CODE or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share one dtype, bf16 or fp16")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda or t.device != q.device:
            raise ValueError(f"{name} must be on q's HIP device")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous [B, N, H, d]")
    return B, Nq, Hq, Hkv, Nk, d


def _check_like(name, t, shape, dtype, device):
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or not t.is_contiguous() \
            or t.device != device:
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {tuple(shape)}")


def attn_bwd_ptr(q: int, k: int, v: int, out: int, dout: int, lse: int, dq: int, dk: int,
                 dv: int, delta: int, B: int, Hq: int, Hkv: int, Nq: int, Nk: int, d: int,
                 scale: float, causal: bool, dtype: int, stream: int = 0) -> int:
    """The C entry point with raw integer pointers; returns the attn_status."""
    return _lib.load().attn_bwd(q or None, k or None, v or None, out or None, dout or None,
                                lse or None, dq or None, dk or None, dv or None, delta or None,
                                int(B), int(Hq), int(Hkv), int(Nq), int(Nk), int(d), float(scale),
                                int(bool(causal)), int(dtype), stream or None)


def attn_bwd_ext_ptr(q: int, k: int, v: int, out: int, dout: int, lse: int, dq: int, dk: int,
                     dv: int, delta: int, B: int, Hq: int, Hkv: int, Nq: int, Nk: int, d: int,
                     scale: float, causal: bool, window_left: int, window_right: int,
                     alibi_slopes: int, softcap: float, dtype: int, stream: int = 0) -> int:
    """The C entry point attn_bwd_ext with raw integer pointers."""
    return _lib.load().attn_bwd_ext(q or None, k or None, v or None, out or None, dout or None,
                                    lse or None, dq or None, dk or None, dv or None, delta or None,
                                    int(B), int(Hq), int(Hkv), int(Nq), int(Nk), int(d),
                                    float(scale), int(bool(causal)), int(window_left),
                                    int(window_right), alibi_slopes or None, float(softcap),
                                    int(dtype), stream or None)


def attn_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor,
             dout: torch.Tensor, lse: torch.Tensor, softmax_scale: float | None = None,
             causal: bool = False, window: tuple = (-1, -1),
             alibi_slopes: torch.Tensor | None = None, softcap: float = 0.0):
    """Exact attention backward on the GPU.

    q, out, dout: [B, Nq, Hq, d]; k, v: [B, Nk, Hkv, d]; lse: [B, Hq, Nq] fp32 --
    ``out`` and ``lse`` as returned by ``attn_fwd`` for the same arguments
    (score variants included: ``window``, ``alibi_slopes``, ``softcap`` select
    attn_bwd_ext).
    Returns (dq like q, dk like k, dv like v, delta [B, Hq, Nq] fp32).
    """
    B, Nq, Hq, Hkv, Nk, d = _check_qkv(q, k, v)
    _check_like("out", out, q.shape, q.dtype, q.device)
    _check_like("dout", dout, q.shape, q.dtype, q.device)
    _check_like("lse", lse, (B, Hq, Nq), torch.float32, q.device)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    delta = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    left, right = (int(x) for x in window)
    # Any window other than (-1, -1) goes to the variant entry point, which
    # rejects bounds below -1 with ATTN_ERR_BAD_ARGUMENT.
    variants = (left, right) != (-1, -1) or alibi_slopes is not None or softcap != 0.0
    if alibi_slopes is not None:
        _check_like("alibi_slopes", alibi_slopes, (Hq,), torch.float32, q.device)
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        if variants:
            code = attn_bwd_ext_ptr(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                    dout.data_ptr(), lse.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                                    dv.data_ptr(), delta.data_ptr(), B, Hq, Hkv, Nq, Nk, d,
                                    softmax_scale, causal, left, right,
                                    alibi_slopes.data_ptr() if alibi_slopes is not None else 0,
                                    softcap, _DTYPE_CODE[q.dtype], stream)
        else:
            code = attn_bwd_ptr(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                dout.data_ptr(), lse.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                                dv.data_ptr(), delta.data_ptr(), B, Hq, Hkv, Nq, Nk, d,
                                softmax_scale, causal, _DTYPE_CODE[q.dtype], stream)
    if code != _lib.ATTN_OK:
        raise AttnError(code)
    return dq, dk, dv, delta


def attn_decode_ptr(q: int, k_cache: int, v_cache: int, cache_seqlens: int, k_new: int, v_new: int,
                    out: int, lse: int, workspace: int, workspace_bytes: int, B: int, Hq: int,
                    Hkv: int, Nq: int, Ncap: int, Nnew: int, d: int, scale: float, causal: bool,
                    dtype: int, num_splits: int = 0, stream: int = 0) -> int:
    """The C entry point with raw integer pointers; returns the attn_status."""
    return _lib.load().attn_decode(q or None, k_cache or None, v_cache or None,
                                   cache_seqlens or None, k_new or None, v_new or None,
                                   out or None, lse or None, workspace or None,
                                   int(workspace_bytes), int(B), int(Hq), int(Hkv), int(Nq),
                                   int(Ncap), int(Nnew), int(d), float(scale),
                                   int(bool(causal)), int(dtype), int(num_splits), stream or None)


def attn_decode_num_splits(B: int, Hq: int, Hkv: int, Nq: int, Ncap: int, d: int) -> int:
    return int(_lib.load().attn_decode_num_splits(B, Hq, Hkv, Nq, Ncap, d))


def attn_decode_workspace_size(B: int, Hq: int, Nq: int, d: int, num_splits: int) -> int:
    return int(_lib.load().attn_decode_workspace_size(B, Hq, Nq, d, num_splits))


def attn_decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                cache_seqlens: torch.Tensor, k_new: torch.Tensor | None = None,
                v_new: torch.Tensor | None = None, softmax_scale: float | None = None,
                causal: bool = True, num_splits: int = 0):
    """KV-cache decode forward on the GPU (the caches are updated in place).

    q: [B, Nq, Hq, d]; k_cache, v_cache: [B, Ncap, Hkv, d]; cache_seqlens:
    int32 [B] on the device (rows already in the cache); k_new, v_new:
    [B, Nnew, Hkv, d] or None.  Returns (out [B, Nq, Hq, d], lse [B, Hq, Nq]).
    """
    B, Nq, Hq, Hkv, Ncap, d = _check_qkv(q, k_cache, v_cache)
    _check_like("cache_seqlens", cache_seqlens, (B,), torch.int32, q.device)
    Nnew = 0
    if k_new is not None or v_new is not None:
        if k_new is None or v_new is None:
            raise ValueError("k_new and v_new go together")
        Nnew = k_new.shape[1]
        _check_like("k_new", k_new, (B, Nnew, Hkv, d), q.dtype, q.device)
        _check_like("v_new", v_new, (B, Nnew, Hkv, d), q.dtype, q.device)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    splits = num_splits or attn_decode_num_splits(B, Hq, Hkv, Nq, Ncap, d)
    ws_bytes = attn_decode_workspace_size(B, Hq, Nq, d, splits)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=q.device)
    out = torch.empty_like(q)
    lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        code = attn_decode_ptr(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                               cache_seqlens.data_ptr(),
                               k_new.data_ptr() if Nnew else 0, v_new.data_ptr() if Nnew else 0,
                               out.data_ptr(), lse.data_ptr(), ws.data_ptr(), ws_bytes, B, Hq, Hkv,
                               Nq, Ncap, Nnew, d, softmax_scale, causal, _DTYPE_CODE[q.dtype],
                               splits, stream)
    if code != _lib.ATTN_OK:
        raise AttnError(code)
    return out, lse


def attn_decode_noalloc_ptr(q: int, k_cache: int, v_cache: int, cache_seqlens: int, k_new: int,
                            v_new: int, out: int, lse: int, B: int, Hq: int, Hkv: int, Nq: int,
                            Ncap: int, Nnew: int, d: int, scale: float, causal: bool, dtype: int,
                            num_splits: int = 0, stream: int = 0) -> int:
    """attn_decode_noalloc with raw integer pointers; returns the attn_status."""
    return _lib.load().attn_decode_noalloc(q or None, k_cache or None, v_cache or None,
                                           cache_seqlens or None, k_new or None, v_new or None,
                                           out or None, lse or None, int(B), int(Hq), int(Hkv),
                                           int(Nq), int(Ncap), int(Nnew), int(d), float(scale),
                                           int(bool(causal)), int(dtype), int(num_splits),
                                           stream or None)


def attn_decode_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                        cache_seqlens: torch.Tensor, k_new: torch.Tensor | None = None,
                        v_new: torch.Tensor | None = None, softmax_scale: float | None = None,
                        causal: bool = True, num_splits: int = 0, out: torch.Tensor | None = None,
                        lse: torch.Tensor | None = None):
    """``attn_decode`` through the entry point that allocates nothing: the
    split partials live in the library's own per-GPU scratch array.  Pass
    ``out`` and ``lse`` to keep this call free of allocations as well (they
    are allocated here otherwise).  Returns (out, lse)."""
    B, Nq, Hq, Hkv, Ncap, d = _check_qkv(q, k_cache, v_cache)
    _check_like("cache_seqlens", cache_seqlens, (B,), torch.int32, q.device)
    Nnew = 0
    if k_new is not None or v_new is not None:
        if k_new is None or v_new is None:
            raise ValueError("k_new and v_new go together")
        Nnew = k_new.shape[1]
        _check_like("k_new", k_new, (B, Nnew, Hkv, d), q.dtype, q.device)
        _check_like("v_new", v_new, (B, Nnew, Hkv, d), q.dtype, q.device)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    _check_like("out", out, tuple(q.shape), q.dtype, q.device)
    _check_like("lse", lse, (B, Hq, Nq), torch.float32, q.device)
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        code = attn_decode_noalloc_ptr(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                       cache_seqlens.data_ptr(),
                                       k_new.data_ptr() if Nnew else 0,
                                       v_new.data_ptr() if Nnew else 0, out.data_ptr(),
                                       lse.data_ptr(), B, Hq, Hkv, Nq, Ncap, Nnew, d,
                                       softmax_scale, causal, _DTYPE_CODE[q.dtype], num_splits,
                                       stream)
    if code != _lib.ATTN_OK:
        raise AttnError(code)
    return out, lse


def attn_fwd_varlen_ptr(q: int, k: int, v: int, out: int, lse: int, cu_q: int, cu_k: int, B: int,
                        Hq: int, Hkv: int, total_q: int, total_k: int, max_seqlen_q: int, d: int,
                        scale: float, causal: bool, dtype: int, stream: int = 0) -> int:
    """The C entry point attn_fwd_varlen with raw integer pointers."""
    return _lib.load().attn_fwd_varlen(q or None, k or None, v or None, out or None, lse or None,
                                       cu_q or None, cu_k or None, int(B), int(Hq), int(Hkv),
                                       int(total_q), int(total_k), int(max_seqlen_q), int(d),
                                       float(scale), int(bool(causal)), int(dtype), stream or None)


def attn_fwd_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                    cu_seqlens_q: torch.Tensor, cu_seqlens_k: torch.Tensor, max_seqlen_q: int,
                    softmax_scale: float | None = None, causal: bool = False):
    """Exact attention over packed variable-length sequences.

    q: [total_q, Hq, d]; k, v: [total_k, Hkv, d]; cu_seqlens_*: int32 [B + 1]
    on the device.  Returns (out [total_q, Hq, d], lse [Hq, total_q] fp32).
    """
    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3:
        raise ValueError("q, k, v must be 3-D [total, H, d]")
    total_q, Hq, d = q.shape
    total_k, Hkv, dk = k.shape
    if tuple(v.shape) != tuple(k.shape) or dk != d:
        raise ValueError("k and v must be [total_k, Hkv, d] with q's d")
    if q.dtype not in _DTYPE_CODE or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share one dtype, bf16 or fp16")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda or t.device != q.device or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous tensor on q's HIP device")
    B = cu_seqlens_q.numel() - 1
    _check_like("cu_seqlens_q", cu_seqlens_q, (B + 1,), torch.int32, q.device)
    _check_like("cu_seqlens_k", cu_seqlens_k, (B + 1,), torch.int32, q.device)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    out = torch.empty_like(q)
    lse = torch.empty((Hq, total_q), dtype=torch.float32, device=q.device)
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        code = attn_fwd_varlen_ptr(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                   lse.data_ptr(), cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr(),
                                   B, Hq, Hkv, total_q, total_k, max_seqlen_q, d, softmax_scale,
                                   causal, _DTYPE_CODE[q.dtype], stream)
    if code != _lib.ATTN_OK:
        raise AttnError(code)
    return out, lse


BLOCK_MASK_SIZE = 128  # rows and keys per block of the block mask (ATTN_BLOCK_MASK_SIZE)


def attn_fwd_blocksparse_ptr(q: int, k: int, v: int, out: int, lse: int, block_mask: int,
                             mask_heads: int, B: int, Hq: int, Hkv: int, Nq: int, Nk: int, d: int,
                             scale: float, causal: bool, dtype: int, stream: int = 0) -> int:
    """The C entry point attn_fwd_blocksparse with raw integer pointers."""
    return _lib.load().attn_fwd_blocksparse(q or None, k or None, v or None, out or None,
                                            lse or None, block_mask or None, int(mask_heads),
                                            int(B), int(Hq), int(Hkv), int(Nq), int(Nk), int(d),
                                            float(scale), int(bool(causal)), int(dtype),
                                            stream or None)


def attn_fwd_blocksparse(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                         block_mask: torch.Tensor, softmax_scale: float | None = None,
                         causal: bool = False, out: torch.Tensor | None = None,
                         lse: torch.Tensor | None = None):
    """Exact attention restricted by a block mask.

    q: [B, Nq, Hq, d]; k, v: [B, Nk, Hkv, d] as for ``attn_fwd``; block_mask:
    uint8 or bool [B, 1 or Hq, ceil(Nq / 128), ceil(Nk / 128)] on q's device,
    nonzero where a (query block, key block) pair of 128 x 128 takes part.
    Returns (out [B, Nq, Hq, d], lse [B, Hq, Nq] fp32).
    """
    B, Nq, Hq, Hkv, Nk, d = _check_qkv(q, k, v)
    nqb, nkb = -(-Nq // BLOCK_MASK_SIZE), -(-Nk // BLOCK_MASK_SIZE)
    if block_mask.dtype == torch.bool:
        block_mask = block_mask.view(torch.uint8)
    if block_mask.dim() != 4 or block_mask.shape[1] not in (1, Hq):
        raise ValueError(f"block_mask must be [B, 1 or Hq, {nqb}, {nkb}]")
    _check_like("block_mask", block_mask, (B, block_mask.shape[1], nqb, nkb), torch.uint8, q.device)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    _check_like("out", out, q.shape, q.dtype, q.device)
    _check_like("lse", lse, (B, Hq, Nq), torch.float32, q.device)
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        code = attn_fwd_blocksparse_ptr(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                        lse.data_ptr(), block_mask.data_ptr(), block_mask.shape[1],
                                        B, Hq, Hkv, Nq, Nk, d, softmax_scale, causal,
                                        _DTYPE_CODE[q.dtype], stream)
    if code != _lib.ATTN_OK:
        raise AttnError(code)
    return out, lse


def attn_bwd_blocksparse_ptr(q: int, k: int, v: int, out: int, dout: int, lse: int, dq: int,
                             dk: int, dv: int, delta: int, block_mask: int, mask_heads: int,
                             B: int, Hq: int, Hkv: int, Nq: int, Nk: int, d: int, scale: float,
                             causal: bool, dtype: int, stream: int = 0) -> int:
    """The C entry point attn_bwd_blocksparse with raw integer pointers."""
    return _lib.load().attn_bwd_blocksparse(
        q or None, k or None, v or None, out or None, dout or None, lse or None, dq or None,
        dk or None, dv or None, delta or None, block_mask or None, int(mask_heads), int(B),
        int(Hq), int(Hkv), int(Nq), int(Nk), int(d), float(scale), int(bool(causal)), int(dtype),
        stream or None)


def attn_bwd_blocksparse(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor,
                         dout: torch.Tensor, lse: torch.Tensor, block_mask: torch.Tensor,
                         softmax_scale: float | None = None, causal: bool = False):
    """Backward of ``attn_fwd_blocksparse``: ``out`` and ``lse`` as it returned
    them for the same arguments and mask.  Returns (dq, dk, dv, delta)."""
    B, Nq, Hq, Hkv, Nk, d = _check_qkv(q, k, v)
    _check_like("out", out, q.shape, q.dtype, q.device)
    _check_like("dout", dout, q.shape, q.dtype, q.device)
    _check_like("lse", lse, (B, Hq, Nq), torch.float32, q.device)
    nqb, nkb = -(-Nq // BLOCK_MASK_SIZE), -(-Nk // BLOCK_MASK_SIZE)
    if block_mask.dtype == torch.bool:
        block_mask = block_mask.view(torch.uint8)
    if block_mask.dim() != 4 or block_mask.shape[1] not in (1, Hq):
        raise ValueError(f"block_mask must be [B, 1 or Hq, {nqb}, {nkb}]")
    _check_like("block_mask", block_mask, (B, block_mask.shape[1], nqb, nkb), torch.uint8, q.device)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    delta = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        code = attn_bwd_blocksparse_ptr(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                        dout.data_ptr(), lse.data_ptr(), dq.data_ptr(),
                                        dk.data_ptr(), dv.data_ptr(), delta.data_ptr(),
                                        block_mask.data_ptr(), block_mask.shape[1], B, Hq, Hkv,
                                        Nq, Nk, d, softmax_scale, causal, _DTYPE_CODE[q.dtype],
                                        stream)
    if code != _lib.ATTN_OK:
        raise AttnError(code)
    return dq, dk, dv, delta


def attn_bwd_varlen_ptr(q: int, k: int, v: int, out: int, dout: int, lse: int, dq: int, dk: int,
                        dv: int, delta: int, cu_q: int, cu_k: int, B: int, Hq: int, Hkv: int,
                        total_q: int, total_k: int, max_seqlen_q: int, max_seqlen_k: int, d: int,
                        scale: float, causal: bool, dtype: int, stream: int = 0) -> int:
    """The C entry point attn_bwd_varlen with raw integer pointers."""
    return _lib.load().attn_bwd_varlen(
        q or None, k or None, v or None, out or None, dout or None, lse or None, dq or None,
        dk or None, dv or None, delta or None, cu_q or None, cu_k or None, int(B), int(Hq),
        int(Hkv), int(total_q), int(total_k), int(max_seqlen_q), int(max_seqlen_k), int(d),
        float(scale), int(bool(causal)), int(dtype), stream or None)


def attn_bwd_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor,
                    dout: torch.Tensor, lse: torch.Tensor, cu_seqlens_q: torch.Tensor,
                    cu_seqlens_k: torch.Tensor, max_seqlen_q: int, max_seqlen_k: int,
                    softmax_scale: float | None = None, causal: bool = False):
    """Backward of ``attn_fwd_varlen``: q, out, dout [total_q, Hq, d]; k, v
    [total_k, Hkv, d]; lse [Hq, total_q] as the forward returned it.
    Returns (dq, dk, dv, delta [Hq, total_q])."""
    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3:
        raise ValueError("q, k, v must be 3-D [total, H, d]")
    total_q, Hq, d = q.shape
    total_k, Hkv, dk_ = k.shape
    if tuple(v.shape) != tuple(k.shape) or dk_ != d:
        raise ValueError("k and v must be [total_k, Hkv, d] with q's d")
    if q.dtype not in _DTYPE_CODE or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share one dtype, bf16 or fp16")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda or t.device != q.device or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous tensor on q's HIP device")
    _check_like("out", out, q.shape, q.dtype, q.device)
    _check_like("dout", dout, q.shape, q.dtype, q.device)
    _check_like("lse", lse, (Hq, total_q), torch.float32, q.device)
    B = cu_seqlens_q.numel() - 1
    _check_like("cu_seqlens_q", cu_seqlens_q, (B + 1,), torch.int32, q.device)
    _check_like("cu_seqlens_k", cu_seqlens_k, (B + 1,), torch.int32, q.device)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    delta = torch.empty((Hq, total_q), dtype=torch.float32, device=q.device)
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        code = attn_bwd_varlen_ptr(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                   dout.data_ptr(), lse.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                                   dv.data_ptr(), delta.data_ptr(), cu_seqlens_q.data_ptr(),
                                   cu_seqlens_k.data_ptr(), B, Hq, Hkv, total_q, total_k,
                                   max_seqlen_q, max_seqlen_k, d, softmax_scale, causal,
                                   _DTYPE_CODE[q.dtype], stream)
    if code != _lib.ATTN_OK:
        raise AttnError(code)
    return dq, dk, dv, delta


class _Attention(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, softmax_scale, causal, window, alibi_slopes, softcap):
        out, lse = attn_fwd(q, k, v, softmax_scale, causal, window=window,
                            alibi_slopes=alibi_slopes, softcap=softcap)
        # The slopes are saved like the tensors, so that autograd's version
        # check catches an in-place change between the forward and backward.
        extra = (alibi_slopes,) if alibi_slopes is not None else ()
        ctx.save_for_backward(q, k, v, out, lse, *extra)
        ctx.softmax_scale, ctx.causal = softmax_scale, causal
        ctx.window, ctx.softcap = window, softcap
        return out

    @staticmethod
    def backward(ctx, dout):
        q, k, v, out, lse, *extra = ctx.saved_tensors
        slopes = extra[0] if extra else None
        dq, dk, dv, _ = attn_bwd(q, k, v, out, dout.contiguous(), lse, ctx.softmax_scale, ctx.causal,
                                 window=ctx.window, alibi_slopes=slopes, softcap=ctx.softcap)
        return dq, dk, dv, None, None, None, None, None


def attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
              softmax_scale: float | None = None, causal: bool = False, *,
              window: tuple = (-1, -1), alibi_slopes: torch.Tensor | None = None,
              softcap: float = 0.0) -> torch.Tensor:
    """Exact attention with autograd: ``attn_fwd`` forward, ``attn_bwd``
    backward, with the same score variants (sliding ``window``, ALiBi
    ``alibi_slopes`` [Hq] fp32 -- constants, no gradient -- and ``softcap``)."""
    return _Attention.apply(q, k, v, softmax_scale, causal, tuple(window), alibi_slopes, softcap)


def attn_fwd_ext_ptr(q: int, k: int, v: int, out: int, lse: int, B: int, Hq: int, Hkv: int,
                     Nq: int, Nk: int, d: int, scale: float, causal: bool, window_left: int,
                     window_right: int, alibi_slopes: int, softcap: float, dtype: int,
                     stream: int = 0) -> int:
    """The C entry point attn_fwd_ext with raw integer pointers."""
    return _lib.load().attn_fwd_ext(q or None, k or None, v or None, out or None, lse or None,
                                    int(B), int(Hq), int(Hkv), int(Nq), int(Nk), int(d),
                                    float(scale), int(bool(causal)), int(window_left),
                                    int(window_right), alibi_slopes or None, float(softcap),
                                    int(dtype), stream or None)


def attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, softmax_scale: float | None = None,
             causal: bool = False, out: torch.Tensor | None = None,
             lse: torch.Tensor | None = None, window: tuple = (-1, -1),
             alibi_slopes: torch.Tensor | None = None, softcap: float = 0.0):
    """Exact attention forward on the GPU.

    q: [B, Nq, Hq, d]; k, v: [B, Nk, Hkv, d]; contiguous bf16 or fp16 tensors
    on one HIP device.  ``softmax_scale`` defaults to 1/sqrt(d).  Score
    variants (attn_fwd_ext): ``window`` = (left, right) keys around the
    bottom-right diagonal (-1 = unbounded), ``alibi_slopes`` fp32 [Hq] on the
    device, ``softcap`` > 0.
    Returns (out [B, Nq, Hq, d] of q's dtype, lse [B, Hq, Nq] fp32).
    """
    B, Nq, Hq, Hkv, Nk, d = _check_qkv(q, k, v)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    if out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous() or out.device != q.device:
        raise ValueError("out must be a contiguous tensor like q")
    if tuple(lse.shape) != (B, Hq, Nq) or lse.dtype != torch.float32 or not lse.is_contiguous() \
            or lse.device != q.device:
        raise ValueError("lse must be a contiguous fp32 tensor [B, Hq, Nq]")
    left, right = (int(x) for x in window)
    # Any window other than (-1, -1) goes to the variant entry point, which
    # rejects bounds below -1 with ATTN_ERR_BAD_ARGUMENT.
    variants = (left, right) != (-1, -1) or alibi_slopes is not None or softcap != 0.0
    if alibi_slopes is not None:
        _check_like("alibi_slopes", alibi_slopes, (Hq,), torch.float32, q.device)
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        if variants:
            code = attn_fwd_ext_ptr(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                    lse.data_ptr(), B, Hq, Hkv, Nq, Nk, d, softmax_scale, causal,
                                    left, right,
                                    alibi_slopes.data_ptr() if alibi_slopes is not None else 0,
                                    softcap, _DTYPE_CODE[q.dtype], stream)
        else:
            code = attn_fwd_ptr(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                lse.data_ptr(), B, Hq, Hkv, Nq, Nk, d, softmax_scale, causal,
                                _DTYPE_CODE[q.dtype], stream)
    if code != _lib.ATTN_OK:
        raise AttnError(code)
    return out, lse
