"""Host-side tests of the C ABI (no GPU needed, no kernel is ever launched).

Every call below fails validation before the library makes any HIP call,
except the no-device check, which only runs where no GPU is visible.  The
pointers are fake but 16-byte aligned, and are never dereferenced.
"""

import ctypes
import os
import re

import pytest
import torch

from exact_tiled_attention_35_amd import _lib
from exact_tiled_attention_35_amd.attention import attn_bwd_ptr, attn_fwd_ptr, attn_status_string, attn_version

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# Fake, aligned, non-overlapping "device" addresses (never dereferenced).
Q, K, V, OUT, LSE = 0x10000000, 0x20000000, 0x30000000, 0x40000000, 0x50000000
GOOD = dict(q=Q, k=K, v=V, out=OUT, lse=LSE, B=2, Hq=8, Hkv=2, Nq=100, Nk=120, d=128,
            scale=0.088, causal=True, dtype=_lib.ATTN_DTYPE_BF16)


def call(**over):
    a = dict(GOOD)
    a.update(over)
    return attn_fwd_ptr(a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"], a["Hq"], a["Hkv"],
                        a["Nq"], a["Nk"], a["d"], a["scale"], a["causal"], a["dtype"])


def declared_functions():
    with open(os.path.join(ROOT, "include", "attn.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(attn_\w+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    names = declared_functions()
    assert names == ["attn_bwd", "attn_bwd_blocksparse", "attn_bwd_ext", "attn_bwd_varlen", "attn_decode",
                     "attn_decode_noalloc", "attn_decode_num_splits", "attn_decode_workspace_size",
                     "attn_fwd", "attn_fwd_blocksparse", "attn_fwd_ext", "attn_fwd_varlen",
                     "attn_status_string", "attn_version"]
    for n in names:
        assert hasattr(lib, n), n
        assert ctypes.cast(getattr(lib, n), ctypes.c_void_p).value


def test_version_and_messages():
    assert "gfx950" in attn_version()
    codes = [0, -1, -2, -3, -4, -5, -6, -7, -8, -9, -10, -11, -12, -13]
    msgs = [attn_status_string(c) for c in codes]
    assert len(set(msgs)) == len(codes)
    assert msgs[0].startswith("ATTN_OK")
    assert attn_status_string(12345) == "unknown attn status"


@pytest.mark.parametrize("field,value", [("B", -1), ("Nq", -1), ("Hq", 0), ("Hkv", 0), ("Nk", 0), ("d", 0)])
def test_bad_shape(field, value):
    assert call(**{field: value}) == _lib.ATTN_ERR_BAD_SHAPE


def test_too_large_is_bad_shape():
    assert call(B=1 << 30, Nq=1 << 30, Hq=1 << 8, Hkv=1, d=256) == _lib.ATTN_ERR_BAD_SHAPE
    # a head count whose 128-row q window exceeds 32-bit byte offsets
    assert call(Hq=1 << 16, Hkv=1 << 16, d=128) == _lib.ATTN_ERR_BAD_SHAPE
    # too many workgroups for one grid
    assert call(B=1 << 16, Hq=1 << 10, Hkv=1, Nq=1 << 20, d=64) == _lib.ATTN_ERR_BAD_SHAPE


@pytest.mark.parametrize("field", ["B", "Nq"])
def test_empty_problem_is_a_noop_even_with_null_pointers(field):
    assert call(**{field: 0}, q=0, k=0, v=0, out=0, lse=0, dtype=99, d=7) == _lib.ATTN_OK


def test_shape_is_checked_before_empty():
    assert call(B=0, Nk=0) == _lib.ATTN_ERR_BAD_SHAPE


@pytest.mark.parametrize("field", ["q", "k", "v", "out", "lse"])
def test_null_pointer(field):
    assert call(**{field: 0}) == _lib.ATTN_ERR_NULL_POINTER


def test_gqa_ratio():
    assert call(Hq=8, Hkv=3) == _lib.ATTN_ERR_GQA_RATIO
    assert call(Hq=2, Hkv=4) == _lib.ATTN_ERR_GQA_RATIO


@pytest.mark.parametrize("d", [1, 32, 96, 100, 192, 512])
def test_unsupported_head_dim(d):
    assert call(d=d) == _lib.ATTN_ERR_UNSUPPORTED_HDIM


@pytest.mark.parametrize("dtype", [-1, 2, 7])
def test_unsupported_dtype(dtype):
    assert call(dtype=dtype) == _lib.ATTN_ERR_UNSUPPORTED_DTYPE


@pytest.mark.parametrize("scale", [float("nan"), float("inf"), float("-inf"), 1e39])
def test_bad_scale(scale):
    # 1e39 overflows to +inf when narrowed to the ABI's fp32.
    assert call(scale=scale) == _lib.ATTN_ERR_BAD_SCALE


@pytest.mark.parametrize("field", ["q", "k", "v", "out", "lse"])
def test_misaligned(field):
    assert call(**{field: GOOD[field] + 8}) == _lib.ATTN_ERR_MISALIGNED


def test_aliasing():
    # out overlapping q, lse overlapping v, out overlapping lse, in-place out == q
    assert call(out=Q) == _lib.ATTN_ERR_ALIASING
    assert call(lse=V + 64) == _lib.ATTN_ERR_ALIASING
    assert call(lse=OUT + 16) == _lib.ATTN_ERR_ALIASING
    assert call(out=K - 16) == _lib.ATTN_ERR_ALIASING


def test_validation_order():
    # null pointer reported before the GQA ratio, GQA before head dim, ...
    assert call(q=0, Hkv=3) == _lib.ATTN_ERR_NULL_POINTER
    assert call(Hkv=3, d=100) == _lib.ATTN_ERR_GQA_RATIO
    assert call(d=100, dtype=9) == _lib.ATTN_ERR_UNSUPPORTED_HDIM
    assert call(dtype=9, scale=float("nan")) == _lib.ATTN_ERR_UNSUPPORTED_DTYPE
    assert call(scale=float("nan"), q=Q + 2) == _lib.ATTN_ERR_BAD_SCALE
    assert call(q=Q + 2, out=Q) == _lib.ATTN_ERR_MISALIGNED


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="a HIP device is visible here")
def test_no_device_reported_without_gpu():
    assert call() == _lib.ATTN_ERR_NO_DEVICE
    assert call(causal=False, dtype=_lib.ATTN_DTYPE_F16, d=64) == _lib.ATTN_ERR_NO_DEVICE


def test_python_binding_rejects_bad_tensors():
    from exact_tiled_attention_35_amd import attn_fwd

    q = torch.zeros(1, 4, 2, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        attn_fwd(q, q[:, :, :1], q, causal=False)  # k/v shape mismatch
    with pytest.raises(ValueError):
        attn_fwd(q.float(), q.float(), q.float())  # fp32 is not an ABI dtype
    with pytest.raises(ValueError):
        attn_fwd(q, q, q)  # CPU tensors


# ---------------------------------------------------------------------------
# attn_bwd
# ---------------------------------------------------------------------------
OUT_, DOUT, DQ, DK, DV, DELTA = 0x60000000, 0x70000000, 0x80000000, 0x90000000, 0xA0000000, 0xB0000000
GOOD_BWD = dict(q=Q, k=K, v=V, out=OUT_, dout=DOUT, lse=LSE, dq=DQ, dk=DK, dv=DV, delta=DELTA,
                B=2, Hq=8, Hkv=2, Nq=100, Nk=120, d=128, scale=0.088, causal=True,
                dtype=_lib.ATTN_DTYPE_BF16)
BWD_ORDER = ["q", "k", "v", "out", "dout", "lse", "dq", "dk", "dv", "delta",
             "B", "Hq", "Hkv", "Nq", "Nk", "d", "scale", "causal", "dtype"]


def call_bwd(**over):
    a = dict(GOOD_BWD)
    a.update(over)
    return attn_bwd_ptr(*[a[n] for n in BWD_ORDER])


@pytest.mark.parametrize("field,value", [("B", -1), ("Nq", -1), ("Hq", 0), ("Hkv", 0), ("Nk", 0), ("d", 0)])
def test_bwd_bad_shape(field, value):
    assert call_bwd(**{field: value}) == _lib.ATTN_ERR_BAD_SHAPE


def test_bwd_too_large_is_bad_shape():
    assert call_bwd(B=1 << 30, Nq=1 << 30, Hq=1 << 8, Hkv=1, d=256) == _lib.ATTN_ERR_BAD_SHAPE
    assert call_bwd(Hq=1 << 16, Hkv=1 << 16, d=128) == _lib.ATTN_ERR_BAD_SHAPE


def test_bwd_empty_batch_is_a_noop_with_null_pointers():
    nulls = {n: 0 for n in BWD_ORDER[:10]}
    assert call_bwd(B=0, dtype=99, d=7, **nulls) == _lib.ATTN_OK


@pytest.mark.parametrize("field", ["q", "k", "v", "out", "dout", "lse", "dq", "dk", "dv", "delta"])
def test_bwd_null_pointer(field):
    assert call_bwd(**{field: 0}) == _lib.ATTN_ERR_NULL_POINTER


@pytest.mark.parametrize("field", ["q", "out", "dout", "lse", "dq", "delta"])
def test_bwd_no_query_rows_allows_null_row_buffers(field):
    # Nq == 0 passes validation with these NULL and fails later only for the
    # missing device; k, v, dk and dv stay required.
    code = call_bwd(Nq=0, **{field: 0})
    assert code in (_lib.ATTN_ERR_NO_DEVICE, _lib.ATTN_OK)
    assert call_bwd(Nq=0, dk=0) == _lib.ATTN_ERR_NULL_POINTER


def test_bwd_validation_order():
    assert call_bwd(q=0, Hkv=3) == _lib.ATTN_ERR_NULL_POINTER
    assert call_bwd(Hkv=3, d=100) == _lib.ATTN_ERR_GQA_RATIO
    assert call_bwd(d=100, dtype=9) == _lib.ATTN_ERR_UNSUPPORTED_HDIM
    assert call_bwd(dtype=9, scale=float("inf")) == _lib.ATTN_ERR_UNSUPPORTED_DTYPE
    assert call_bwd(scale=float("nan"), dq=DQ + 4) == _lib.ATTN_ERR_BAD_SCALE
    assert call_bwd(dq=DQ + 4, dk=Q) == _lib.ATTN_ERR_MISALIGNED


@pytest.mark.parametrize("field", ["q", "k", "v", "out", "dout", "lse", "dq", "dk", "dv", "delta"])
def test_bwd_misaligned(field):
    assert call_bwd(**{field: GOOD_BWD[field] + 8}) == _lib.ATTN_ERR_MISALIGNED


def test_bwd_aliasing():
    assert call_bwd(dq=Q) == _lib.ATTN_ERR_ALIASING          # output over an input
    assert call_bwd(dk=V + 16) == _lib.ATTN_ERR_ALIASING
    assert call_bwd(delta=LSE) == _lib.ATTN_ERR_ALIASING
    assert call_bwd(dv=DK) == _lib.ATTN_ERR_ALIASING         # two outputs
    assert call_bwd(delta=DQ + 64) == _lib.ATTN_ERR_ALIASING
    # inputs may share memory (k and v both views of one buffer, say)
    assert call_bwd(v=K) in (_lib.ATTN_ERR_NO_DEVICE, _lib.ATTN_OK)


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="a HIP device is visible here")
def test_bwd_no_device_reported_without_gpu():
    assert call_bwd() == _lib.ATTN_ERR_NO_DEVICE
    assert call_bwd(causal=False, dtype=_lib.ATTN_DTYPE_F16, d=64) == _lib.ATTN_ERR_NO_DEVICE


def test_python_binding_rejects_bad_backward_tensors():
    from exact_tiled_attention_35_amd import attn_bwd

    q = torch.zeros(1, 4, 2, 64, dtype=torch.bfloat16)
    lse = torch.zeros(1, 2, 4)
    with pytest.raises(ValueError):
        attn_bwd(q, q, q, q, q, lse)  # CPU tensors


# ---------------------------------------------------------------------------
# attn_decode
# ---------------------------------------------------------------------------
from exact_tiled_attention_35_amd.attention import (  # noqa: E402
    attn_decode_num_splits, attn_decode_ptr, attn_decode_workspace_size)

KC, VC, SEQ, KN, VN, WS = 0x100000000, 0x200000000, 0x300000000, 0x400000000, 0x500000000, 0x600000000
GOOD_DEC = dict(q=Q, k_cache=KC, v_cache=VC, cache_seqlens=SEQ, k_new=KN, v_new=VN, out=OUT, lse=LSE,
                workspace=WS, workspace_bytes=1 << 30, B=4, Hq=16, Hkv=4, Nq=2, Ncap=4096, Nnew=1,
                d=128, scale=0.088, causal=True, dtype=_lib.ATTN_DTYPE_BF16, num_splits=4)
DEC_ORDER = ["q", "k_cache", "v_cache", "cache_seqlens", "k_new", "v_new", "out", "lse", "workspace",
             "workspace_bytes", "B", "Hq", "Hkv", "Nq", "Ncap", "Nnew", "d", "scale", "causal", "dtype",
             "num_splits"]


def call_dec(**over):
    a = dict(GOOD_DEC)
    a.update(over)
    return attn_decode_ptr(*[a[n] for n in DEC_ORDER])


def test_decode_split_heuristic_and_workspace_size():
    # enough workgroups for two per CU, at least four 32-key tiles per split
    assert attn_decode_num_splits(16, 32, 8, 1, 32768, 128) == 4
    assert attn_decode_num_splits(1, 8, 8, 16, 4096, 128) == 32
    assert attn_decode_num_splits(64, 64, 8, 1, 512, 128) == 1
    assert attn_decode_num_splits(1, 1, 1, 1, 64, 128) == 1
    assert attn_decode_workspace_size(16, 32, 1, 128, 1) == 0
    assert attn_decode_workspace_size(16, 32, 1, 128, 4) == 4 * 16 * 32 * 1 * (128 + 1) * 4


@pytest.mark.parametrize("field,value", [("B", -1), ("Nq", -1), ("Hq", 0), ("Hkv", 0), ("Ncap", 0),
                                         ("Nnew", -1), ("Nnew", 5000), ("d", 0), ("num_splits", -1),
                                         ("num_splits", 129)])
def test_decode_bad_shape(field, value):
    assert call_dec(**{field: value}) == _lib.ATTN_ERR_BAD_SHAPE


def test_decode_noops():
    nulls = {n: 0 for n in DEC_ORDER[:9]}
    assert call_dec(B=0, **nulls) == _lib.ATTN_OK
    assert call_dec(Nq=0, Nnew=0, **nulls) == _lib.ATTN_OK


@pytest.mark.parametrize("field", ["q", "k_cache", "v_cache", "cache_seqlens", "k_new", "v_new",
                                   "out", "lse", "workspace"])
def test_decode_null_pointer(field):
    assert call_dec(**{field: 0}) == _lib.ATTN_ERR_NULL_POINTER


# Calls that pass validation reach the device check: where a GPU is visible
# they would launch kernels on the fake addresses, so they run on GPU-less
# hosts only.
NO_GPU = torch.cuda.device_count() == 0
needs_no_gpu = pytest.mark.skipif(not NO_GPU, reason="would launch kernels on fake addresses")


@needs_no_gpu
def test_decode_optional_pointers():
    # no new rows: k_new / v_new may be NULL; one split: no workspace needed
    assert call_dec(Nnew=0, k_new=0, v_new=0) in (_lib.ATTN_ERR_NO_DEVICE, _lib.ATTN_OK)
    assert call_dec(num_splits=1, workspace=0, workspace_bytes=0) in (_lib.ATTN_ERR_NO_DEVICE, _lib.ATTN_OK)
    # append only (Nq == 0): q, out, lse and the workspace are not needed
    assert call_dec(Nq=0, q=0, out=0, lse=0, workspace=0, workspace_bytes=0) in (
        _lib.ATTN_ERR_NO_DEVICE, _lib.ATTN_OK)


@needs_no_gpu
def test_decode_workspace_too_small():
    need = attn_decode_workspace_size(4, 16, 2, 128, 4)
    assert call_dec(workspace_bytes=need - 1) == _lib.ATTN_ERR_WORKSPACE
    assert call_dec(workspace_bytes=need) in (_lib.ATTN_ERR_NO_DEVICE, _lib.ATTN_OK)


@needs_no_gpu
def test_decode_validation_order_and_alignment():
    assert call_dec(q=0, Hkv=3) == _lib.ATTN_ERR_NULL_POINTER
    assert call_dec(Hkv=3, d=100) == _lib.ATTN_ERR_GQA_RATIO
    assert call_dec(d=100, dtype=5) == _lib.ATTN_ERR_UNSUPPORTED_HDIM
    assert call_dec(dtype=5, scale=float("nan")) == _lib.ATTN_ERR_UNSUPPORTED_DTYPE
    assert call_dec(scale=float("nan"), workspace_bytes=0) == _lib.ATTN_ERR_BAD_SCALE
    assert call_dec(workspace_bytes=0, k_cache=KC + 8) == _lib.ATTN_ERR_WORKSPACE
    assert call_dec(k_cache=KC + 8) == _lib.ATTN_ERR_MISALIGNED
    assert call_dec(cache_seqlens=SEQ + 2) == _lib.ATTN_ERR_MISALIGNED
    assert call_dec(cache_seqlens=SEQ + 4) in (_lib.ATTN_ERR_NO_DEVICE, _lib.ATTN_OK)


def test_decode_aliasing():
    assert call_dec(out=KC) == _lib.ATTN_ERR_ALIASING          # out over the cache
    assert call_dec(k_new=VC + 64) == _lib.ATTN_ERR_ALIASING   # new rows inside a cache
    assert call_dec(workspace=Q) == _lib.ATTN_ERR_ALIASING
    assert call_dec(v_cache=KC + 1024) == _lib.ATTN_ERR_ALIASING


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="a HIP device is visible here")
def test_decode_no_device_reported_without_gpu():
    assert call_dec() == _lib.ATTN_ERR_NO_DEVICE


# ---------------------------------------------------------------------------
# attn_decode_noalloc (no workspace argument; the library's scratch array)
# ---------------------------------------------------------------------------
from exact_tiled_attention_35_amd.attention import attn_decode_noalloc_ptr  # noqa: E402

NOALLOC_ORDER = [n for n in DEC_ORDER if n not in ("workspace", "workspace_bytes")]


def call_noalloc(**over):
    a = dict(GOOD_DEC)
    a.update(over)
    return attn_decode_noalloc_ptr(*[a[n] for n in NOALLOC_ORDER])


def test_noalloc_scratch_size_is_the_declared_one():
    with open(os.path.join(ROOT, "include", "attn.h")) as f:
        m = re.search(r"#define ATTN_DECODE_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", f.read())
    assert m and int(m.group(1)) << int(m.group(2)) == _lib.ATTN_DECODE_SCRATCH_BYTES == 8 << 20


@pytest.mark.parametrize("field,value", [("B", -1), ("Nq", -1), ("Hq", 0), ("Ncap", 0),
                                         ("Nnew", 5000), ("num_splits", 129)])
def test_noalloc_bad_shape(field, value):
    assert call_noalloc(**{field: value}) == _lib.ATTN_ERR_BAD_SHAPE


def test_noalloc_noops():
    nulls = {n: 0 for n in NOALLOC_ORDER[:8]}
    assert call_noalloc(B=0, **nulls) == _lib.ATTN_OK
    assert call_noalloc(Nq=0, Nnew=0, **nulls) == _lib.ATTN_OK


@pytest.mark.parametrize("field", ["q", "k_cache", "v_cache", "cache_seqlens", "k_new", "v_new",
                                   "out", "lse"])
def test_noalloc_null_pointer(field):
    assert call_noalloc(**{field: 0}) == _lib.ATTN_ERR_NULL_POINTER


def test_noalloc_scratch_limit_before_any_hip_call():
    # partials of 2 splits: 2 * B*Hq*Nq * (d + 1) * 4 bytes against 8 MiB
    per_row = (128 + 1) * 4
    fits = (8 << 20) // (2 * per_row)  # 8128 rows of (batch, head, query)
    big = dict(B=1, Hq=fits + 1, Hkv=1, Nq=1, num_splits=2, Nnew=0)
    assert call_noalloc(**big) == _lib.ATTN_ERR_SCRATCH_LIMIT
    assert call_noalloc(**dict(big, num_splits=64)) == _lib.ATTN_ERR_SCRATCH_LIMIT
    # the limit is checked in the workspace step of the documented order
    assert call_noalloc(**dict(big, scale=float("nan"))) == _lib.ATTN_ERR_BAD_SCALE
    assert call_noalloc(**dict(big, k_cache=KC + 8)) == _lib.ATTN_ERR_SCRATCH_LIMIT
    assert "8 MiB" in attn_status_string(_lib.ATTN_ERR_SCRATCH_LIMIT)


@needs_no_gpu
def test_noalloc_fitting_sizes_pass_validation():
    per_row = (128 + 1) * 4
    fits = (8 << 20) // (2 * per_row)
    assert call_noalloc(B=1, Hq=fits, Hkv=1, Nq=1, num_splits=2, Nnew=0) == _lib.ATTN_ERR_NO_DEVICE
    # the library's choice is lowered to what fits instead of failing: here
    # 32 splits (16.9 MB of partials) for attn_decode
    assert attn_decode_num_splits(1, 64, 8, 16, 4096, 128) == 32
    assert attn_decode_workspace_size(1, 64, 16, 128, 32) > (8 << 20)
    assert call_noalloc(B=1, Hq=64, Hkv=8, Nq=16, Ncap=4096, num_splits=0) == _lib.ATTN_ERR_NO_DEVICE
    assert call_noalloc(B=1, Hq=64, Hkv=8, Nq=16, Ncap=4096, num_splits=32) == _lib.ATTN_ERR_SCRATCH_LIMIT
    # one split needs no scratch
    assert call_noalloc(B=64, Hq=64, Hkv=8, Nq=16, num_splits=1) == _lib.ATTN_ERR_NO_DEVICE
    assert call_noalloc(k_cache=KC + 8) == _lib.ATTN_ERR_MISALIGNED
    assert call_noalloc(out=KC) == _lib.ATTN_ERR_ALIASING


# ---------------------------------------------------------------------------
# attn_fwd_ext (score variants)
# ---------------------------------------------------------------------------
from exact_tiled_attention_35_amd.attention import attn_fwd_ext_ptr  # noqa: E402

SLOPES = 0x700000000


def call_ext(left=-1, right=-1, slopes=0, cap=0.0, **over):
    a = dict(GOOD)
    a.update(over)
    return attn_fwd_ext_ptr(a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"], a["Hq"], a["Hkv"],
                            a["Nq"], a["Nk"], a["d"], a["scale"], a["causal"], left, right, slopes,
                            cap, a["dtype"])


def test_ext_without_variants_validates_like_attn_fwd():
    assert call_ext(q=0) == _lib.ATTN_ERR_NULL_POINTER
    assert call_ext() == call()
    assert call_ext(Hkv=3) == _lib.ATTN_ERR_GQA_RATIO
    assert call_ext(B=0, q=0) == _lib.ATTN_OK


@pytest.mark.parametrize("args", [dict(left=-2), dict(right=-5), dict(cap=-1.0),
                                  dict(cap=float("nan")), dict(cap=float("inf"))])
def test_ext_bad_argument(args):
    assert call_ext(**args) == _lib.ATTN_ERR_BAD_ARGUMENT


def test_ext_order_misaligned_and_aliasing():
    assert call_ext(left=-2, scale=float("nan")) == _lib.ATTN_ERR_BAD_SCALE
    assert call_ext(left=-2, q=Q + 2) == _lib.ATTN_ERR_BAD_ARGUMENT
    assert call_ext(slopes=SLOPES + 2) == _lib.ATTN_ERR_MISALIGNED
    assert call_ext(slopes=OUT + 64) == _lib.ATTN_ERR_ALIASING
    assert call_ext(slopes=LSE) == _lib.ATTN_ERR_ALIASING


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="a HIP device is visible here")
def test_ext_no_device_reported_without_gpu():
    assert call_ext(left=4, right=0, slopes=SLOPES, cap=30.0) == _lib.ATTN_ERR_NO_DEVICE


# ---------------------------------------------------------------------------
# attn_fwd_varlen (packed variable-length sequences)
# ---------------------------------------------------------------------------
from exact_tiled_attention_35_amd.attention import attn_fwd_varlen_ptr  # noqa: E402

CUQ, CUK = 0x800000000, 0x900000000
GOOD_VL = dict(q=Q, k=K, v=V, out=OUT, lse=LSE, cu_q=CUQ, cu_k=CUK, B=3, Hq=8, Hkv=2, total_q=300,
               total_k=500, max_q=200, d=128, scale=0.088, causal=True, dtype=_lib.ATTN_DTYPE_BF16)


def call_vl(**over):
    a = dict(GOOD_VL)
    a.update(over)
    return attn_fwd_varlen_ptr(a["q"], a["k"], a["v"], a["out"], a["lse"], a["cu_q"], a["cu_k"],
                               a["B"], a["Hq"], a["Hkv"], a["total_q"], a["total_k"], a["max_q"],
                               a["d"], a["scale"], a["causal"], a["dtype"])


@pytest.mark.parametrize("field,value", [("B", -1), ("Hq", 0), ("Hkv", 0), ("total_q", -1),
                                         ("total_k", -1), ("max_q", -1), ("d", 0)])
def test_varlen_bad_shape(field, value):
    assert call_vl(**{field: value}) == _lib.ATTN_ERR_BAD_SHAPE


@pytest.mark.parametrize("field", ["B", "total_q", "max_q"])
def test_varlen_empty_is_a_noop_with_null_pointers(field):
    assert call_vl(**{field: 0}, q=0, k=0, v=0, out=0, lse=0, cu_q=0, cu_k=0) == _lib.ATTN_OK


def test_varlen_too_large_is_bad_shape():
    assert call_vl(total_q=2**31 - 1, Hq=2**20, Hkv=2**20, d=64) == _lib.ATTN_ERR_BAD_SHAPE
    assert call_vl(Hq=2**24, Hkv=2**24) == _lib.ATTN_ERR_BAD_SHAPE


@pytest.mark.parametrize("field", ["q", "out", "lse", "cu_q", "cu_k", "k", "v"])
def test_varlen_null_pointer(field):
    assert call_vl(**{field: 0}) == _lib.ATTN_ERR_NULL_POINTER


def test_varlen_keys_may_be_null_without_keys():
    # With no key rows, k and v are never read: validation passes to the
    # device check.
    st = call_vl(total_k=0, k=0, v=0)
    assert st in (_lib.ATTN_ERR_NO_DEVICE, _lib.ATTN_OK)


def test_varlen_checks_in_order():
    assert call_vl(Hkv=3) == _lib.ATTN_ERR_GQA_RATIO
    assert call_vl(d=96) == _lib.ATTN_ERR_UNSUPPORTED_HDIM
    assert call_vl(dtype=7) == _lib.ATTN_ERR_UNSUPPORTED_DTYPE
    assert call_vl(scale=float("inf")) == _lib.ATTN_ERR_BAD_SCALE
    assert call_vl(Hkv=3, d=96) == _lib.ATTN_ERR_GQA_RATIO
    assert call_vl(q=Q + 8) == _lib.ATTN_ERR_MISALIGNED
    assert call_vl(cu_q=CUQ + 2) == _lib.ATTN_ERR_MISALIGNED
    assert call_vl(cu_k=CUK + 1) == _lib.ATTN_ERR_MISALIGNED
    assert call_vl(lse=LSE + 4) == _lib.ATTN_ERR_MISALIGNED


def test_varlen_aliasing():
    assert call_vl(out=Q + 256) == _lib.ATTN_ERR_ALIASING
    assert call_vl(lse=CUQ - 64) == _lib.ATTN_ERR_ALIASING
    assert call_vl(cu_k=OUT + 16) == _lib.ATTN_ERR_ALIASING
    assert call_vl(lse=OUT + 1024) == _lib.ATTN_ERR_ALIASING


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="a HIP device is visible here")
def test_varlen_no_device_reported_without_gpu():
    assert call_vl() == _lib.ATTN_ERR_NO_DEVICE


def test_python_varlen_binding_rejects_bad_tensors():
    from exact_tiled_attention_35_amd import attn_fwd_varlen
    q = torch.zeros(10, 4, 64, dtype=torch.bfloat16)
    cu = torch.tensor([0, 10], dtype=torch.int32)
    with pytest.raises(ValueError):
        attn_fwd_varlen(q[0], q, q, cu, cu, 10)
    with pytest.raises(ValueError):
        attn_fwd_varlen(q, q[:, :, :32], q[:, :, :32], cu, cu, 10)
    with pytest.raises(ValueError):
        attn_fwd_varlen(q, q.half(), q.half(), cu, cu, 10)
    with pytest.raises(ValueError):  # CPU tensors
        attn_fwd_varlen(q, q, q, cu, cu, 10)


# ---------------------------------------------------------------------------
# attn_fwd_blocksparse (block mask over 128 x 128 blocks)
# ---------------------------------------------------------------------------
from exact_tiled_attention_35_amd.attention import attn_fwd_blocksparse_ptr  # noqa: E402

MASK = 0xA00000001  # bytes need no alignment


def call_bs(mask=MASK, mask_heads=1, **over):
    a = dict(GOOD)
    a.update(over)
    return attn_fwd_blocksparse_ptr(a["q"], a["k"], a["v"], a["out"], a["lse"], mask, mask_heads,
                                    a["B"], a["Hq"], a["Hkv"], a["Nq"], a["Nk"], a["d"], a["scale"],
                                    a["causal"], a["dtype"])


@pytest.mark.parametrize("field,value", [("B", -1), ("Nq", -1), ("Hq", 0), ("Hkv", 0), ("Nk", 0), ("d", 0)])
def test_blocksparse_bad_shape(field, value):
    assert call_bs(**{field: value}) == _lib.ATTN_ERR_BAD_SHAPE


@pytest.mark.parametrize("field", ["B", "Nq"])
def test_blocksparse_empty_is_a_noop_with_null_pointers(field):
    assert call_bs(**{field: 0}, q=0, k=0, v=0, out=0, lse=0, mask=0) == _lib.ATTN_OK


@pytest.mark.parametrize("field", ["q", "k", "v", "out", "lse", "mask"])
def test_blocksparse_null_pointer(field):
    over = {"mask": 0} if field == "mask" else {field: 0}
    assert call_bs(**over) == _lib.ATTN_ERR_NULL_POINTER


@pytest.mark.parametrize("heads", [0, 2, 7, -1, 9])
def test_blocksparse_mask_heads_must_be_one_or_hq(heads):
    assert call_bs(mask_heads=heads) == _lib.ATTN_ERR_BAD_ARGUMENT


def test_blocksparse_checks_in_order():
    assert call_bs(Hkv=3, mask_heads=2) == _lib.ATTN_ERR_GQA_RATIO
    assert call_bs(d=96) == _lib.ATTN_ERR_UNSUPPORTED_HDIM
    assert call_bs(dtype=7) == _lib.ATTN_ERR_UNSUPPORTED_DTYPE
    assert call_bs(scale=float("nan"), mask_heads=2) == _lib.ATTN_ERR_BAD_SCALE
    assert call_bs(mask_heads=2, q=Q + 8) == _lib.ATTN_ERR_BAD_ARGUMENT
    assert call_bs(q=Q + 8) == _lib.ATTN_ERR_MISALIGNED
    assert call_bs(mask=OUT + 100) == _lib.ATTN_ERR_ALIASING
    assert call_bs(mask=LSE) == _lib.ATTN_ERR_ALIASING
    # mask bytes: B * heads * ceil(Nq/128) * ceil(Nk/128) = 2 * 8 * 1 * 1 = 16
    assert call_bs(mask=OUT - 16, mask_heads=8) != _lib.ATTN_ERR_ALIASING
    assert call_bs(mask=OUT - 15, mask_heads=8) == _lib.ATTN_ERR_ALIASING


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="a HIP device is visible here")
def test_blocksparse_no_device_reported_without_gpu():
    assert call_bs(mask_heads=8) == _lib.ATTN_ERR_NO_DEVICE


# ---------------------------------------------------------------------------
# attn_bwd_blocksparse
# ---------------------------------------------------------------------------
from exact_tiled_attention_35_amd.attention import attn_bwd_blocksparse_ptr  # noqa: E402

BB_DQ, BB_DK, BB_DV, BB_DELTA, BB_DOUT, BB_OUT = (0xB00000000, 0xC00000000, 0xD00000000, 0xE00000000,
                                                0xF00000000, 0x1000000000)


def call_bbs(mask=MASK, mask_heads=1, **over):
    a = dict(q=Q, k=K, v=V, out=BB_OUT, dout=BB_DOUT, lse=LSE, dq=BB_DQ, dk=BB_DK, dv=BB_DV, delta=BB_DELTA,
             B=2, Hq=8, Hkv=2, Nq=100, Nk=120, d=128, scale=0.088, causal=True,
             dtype=_lib.ATTN_DTYPE_BF16)
    a.update(over)
    return attn_bwd_blocksparse_ptr(a["q"], a["k"], a["v"], a["out"], a["dout"], a["lse"], a["dq"],
                                    a["dk"], a["dv"], a["delta"], mask, mask_heads, a["B"], a["Hq"],
                                    a["Hkv"], a["Nq"], a["Nk"], a["d"], a["scale"], a["causal"],
                                    a["dtype"])


def test_bwd_blocksparse_validation():
    assert call_bbs(B=-1) == _lib.ATTN_ERR_BAD_SHAPE
    assert call_bbs(B=0, q=0, mask=0) == _lib.ATTN_OK
    assert call_bbs(mask=0) == _lib.ATTN_ERR_NULL_POINTER
    assert call_bbs(dq=0) == _lib.ATTN_ERR_NULL_POINTER
    assert call_bbs(Hkv=3) == _lib.ATTN_ERR_GQA_RATIO
    assert call_bbs(d=96) == _lib.ATTN_ERR_UNSUPPORTED_HDIM
    assert call_bbs(scale=float("inf"), mask_heads=3) == _lib.ATTN_ERR_BAD_SCALE
    assert call_bbs(mask_heads=3) == _lib.ATTN_ERR_BAD_ARGUMENT
    assert call_bbs(mask_heads=3, q=Q + 8) == _lib.ATTN_ERR_BAD_ARGUMENT
    assert call_bbs(q=Q + 8) == _lib.ATTN_ERR_MISALIGNED
    assert call_bbs(mask=BB_DQ + 4) == _lib.ATTN_ERR_ALIASING
    assert call_bbs(mask=BB_DELTA, mask_heads=8) == _lib.ATTN_ERR_ALIASING


def test_bwd_blocksparse_without_rows_needs_no_mask():
    # Nq == 0: only dk and dv are written (zeros); the mask is never read
    st = call_bbs(Nq=0, q=0, out=0, dout=0, lse=0, dq=0, delta=0, mask=0)
    assert st in (_lib.ATTN_ERR_NO_DEVICE, _lib.ATTN_OK)


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="a HIP device is visible here")
def test_bwd_blocksparse_no_device_reported_without_gpu():
    assert call_bbs(mask_heads=8) == _lib.ATTN_ERR_NO_DEVICE


# ---------------------------------------------------------------------------
# attn_bwd_varlen
# ---------------------------------------------------------------------------
from exact_tiled_attention_35_amd.attention import attn_bwd_varlen_ptr  # noqa: E402

GOOD_BVL = dict(q=Q, k=K, v=V, out=BB_OUT, dout=BB_DOUT, lse=LSE, dq=BB_DQ, dk=BB_DK, dv=BB_DV,
                delta=BB_DELTA, cu_q=CUQ, cu_k=CUK, B=3, Hq=8, Hkv=2, total_q=300, total_k=500,
                max_q=200, max_k=300, d=128, scale=0.088, causal=True, dtype=_lib.ATTN_DTYPE_BF16)
BVL_ORDER = ["q", "k", "v", "out", "dout", "lse", "dq", "dk", "dv", "delta", "cu_q", "cu_k", "B",
             "Hq", "Hkv", "total_q", "total_k", "max_q", "max_k", "d", "scale", "causal", "dtype"]


def call_bvl(**over):
    a = dict(GOOD_BVL)
    a.update(over)
    return attn_bwd_varlen_ptr(*[a[n] for n in BVL_ORDER])


@pytest.mark.parametrize("field,value", [("B", -1), ("Hq", 0), ("Hkv", 0), ("total_q", -1),
                                         ("total_k", -1), ("max_q", -1), ("max_k", -1), ("d", 0)])
def test_bwd_varlen_bad_shape(field, value):
    assert call_bvl(**{field: value}) == _lib.ATTN_ERR_BAD_SHAPE


def test_bwd_varlen_noops_and_null_pointers():
    nulls = dict(q=0, k=0, v=0, out=0, dout=0, lse=0, dq=0, dk=0, dv=0, delta=0, cu_q=0, cu_k=0)
    assert call_bvl(B=0, **nulls) == _lib.ATTN_OK
    assert call_bvl(total_q=0, total_k=0, **nulls) == _lib.ATTN_OK
    for f in ("q", "out", "dout", "lse", "dq", "delta", "k", "v", "dk", "dv", "cu_q", "cu_k"):
        assert call_bvl(**{f: 0}) == _lib.ATTN_ERR_NULL_POINTER, f
    # a side without rows needs no buffers
    st = call_bvl(total_q=0, q=0, out=0, dout=0, lse=0, dq=0, delta=0)
    assert st in (_lib.ATTN_ERR_NO_DEVICE, _lib.ATTN_OK)
    st = call_bvl(total_k=0, k=0, v=0, dk=0, dv=0)
    assert st in (_lib.ATTN_ERR_NO_DEVICE, _lib.ATTN_OK)


def test_bwd_varlen_checks_in_order():
    assert call_bvl(Hkv=3) == _lib.ATTN_ERR_GQA_RATIO
    assert call_bvl(d=96) == _lib.ATTN_ERR_UNSUPPORTED_HDIM
    assert call_bvl(dtype=7) == _lib.ATTN_ERR_UNSUPPORTED_DTYPE
    assert call_bvl(scale=float("nan")) == _lib.ATTN_ERR_BAD_SCALE
    assert call_bvl(cu_q=CUQ + 2) == _lib.ATTN_ERR_MISALIGNED
    assert call_bvl(dk=BB_DK + 8) == _lib.ATTN_ERR_MISALIGNED
    assert call_bvl(dq=Q) == _lib.ATTN_ERR_ALIASING
    assert call_bvl(delta=CUK) == _lib.ATTN_ERR_ALIASING
    assert call_bvl(dv=BB_DK + 64) == _lib.ATTN_ERR_ALIASING


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="a HIP device is visible here")
def test_bwd_varlen_no_device_reported_without_gpu():
    assert call_bvl() == _lib.ATTN_ERR_NO_DEVICE


# ---------------------------------------------------------------------------
# attn_bwd_ext (score variants in the backward)
# ---------------------------------------------------------------------------
from exact_tiled_attention_35_amd.attention import attn_bwd_ext_ptr  # noqa: E402


def call_bext(left=-1, right=-1, slopes=0, cap=0.0, **over):
    a = dict(q=Q, k=K, v=V, out=BB_OUT, dout=BB_DOUT, lse=LSE, dq=BB_DQ, dk=BB_DK, dv=BB_DV,
             delta=BB_DELTA, B=2, Hq=8, Hkv=2, Nq=100, Nk=120, d=128, scale=0.088, causal=True,
             dtype=_lib.ATTN_DTYPE_BF16)
    a.update(over)
    return attn_bwd_ext_ptr(a["q"], a["k"], a["v"], a["out"], a["dout"], a["lse"], a["dq"], a["dk"],
                            a["dv"], a["delta"], a["B"], a["Hq"], a["Hkv"], a["Nq"], a["Nk"], a["d"],
                            a["scale"], a["causal"], left, right, slopes, cap, a["dtype"])


def test_bwd_ext_validation():
    assert call_bext(B=-1) == _lib.ATTN_ERR_BAD_SHAPE
    assert call_bext(B=0, q=0) == _lib.ATTN_OK
    assert call_bext(dk=0) == _lib.ATTN_ERR_NULL_POINTER
    assert call_bext(Hkv=3) == _lib.ATTN_ERR_GQA_RATIO
    for args in (dict(left=-2), dict(right=-3), dict(cap=-1.0), dict(cap=float("nan"))):
        assert call_bext(**args) == _lib.ATTN_ERR_BAD_ARGUMENT, args
    assert call_bext(left=-2, scale=float("inf")) == _lib.ATTN_ERR_BAD_SCALE
    assert call_bext(left=-2, q=Q + 8) == _lib.ATTN_ERR_BAD_ARGUMENT
    assert call_bext(slopes=SLOPES + 2) == _lib.ATTN_ERR_MISALIGNED
    assert call_bext(slopes=BB_DQ + 64) == _lib.ATTN_ERR_ALIASING
    assert call_bext(slopes=BB_DELTA) == _lib.ATTN_ERR_ALIASING


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="a HIP device is visible here")
def test_bwd_ext_no_device_reported_without_gpu():
    assert call_bext(left=5, right=0, slopes=SLOPES, cap=30.0) == _lib.ATTN_ERR_NO_DEVICE
