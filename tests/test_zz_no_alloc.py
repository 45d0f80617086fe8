"""GPU: attn_decode_noalloc (the entry point that allocates nothing; its split
partials live in the library's per-GPU scratch array) against attn_decode
with a caller-owned workspace, through the C ABI.

Bar: the forward's tolerances (max-abs 1e-2 and mean-abs 1e-3 on out, 1e-3
on lse, -inf rows exactly) between the two entry points, and the appended
cache rows bit for bit.  With the same split count both run the same
kernels on the same inputs, so their outputs are also bitwise equal; with
the library's choice of splits the no-allocation call may use fewer (what
fits the scratch), which changes only the order of rounding.  Calls run
back to back, the later ones on smaller inputs, so that a stale partial
left in the shared scratch by an earlier call would show.
"""

import math

import numpy as np
import pytest
import torch

from attn_workloads import make_qkv
from exact_tiled_attention_35_amd import _lib
from exact_tiled_attention_35_amd.attention import (_DTYPE_CODE, attn_decode_noalloc_ptr,
                                                    attn_decode_num_splits, attn_decode_ptr,
                                                    attn_decode_workspace_size)

pytestmark = pytest.mark.gpu

MAX_ABS, MEAN_ABS, LSE_ABS = 1e-2, 1e-3, 1e-3


def make_case(B, Hq, Hkv, Nq, Ncap, lens, Nnew, d, dt, seed):
    q = make_qkv(B, Nq, Nq, Hq, Hq, d, dt, 1.0, seed)[0]
    _, kc, vc = make_qkv(B, 1, Ncap, 1, Hkv, d, dt, 1.0, seed + 1)
    _, kn, vn = make_qkv(B, 1, max(Nnew, 1), 1, Hkv, d, dt, 1.0, seed + 2)
    if Nnew == 0:
        kn = vn = None
    sl = torch.tensor(lens, dtype=torch.int32)
    return q, kc, vc, sl, kn, vn


def run(entry, case, B, Hq, Hkv, Nq, Ncap, Nnew, d, splits):
    """One call on fresh device copies of the inputs; returns (out, lse, k_cache, v_cache) on the CPU."""
    q, kc, vc, sl, kn, vn = (t.cuda() if t is not None else None for t in case)
    out = torch.empty_like(q)
    lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device="cuda")
    scale = 1.0 / math.sqrt(d)
    stream = torch.cuda.current_stream().cuda_stream
    ptrs = [q.data_ptr(), kc.data_ptr(), vc.data_ptr(), sl.data_ptr(),
            kn.data_ptr() if kn is not None else 0, vn.data_ptr() if vn is not None else 0,
            out.data_ptr(), lse.data_ptr()]
    dtc = _DTYPE_CODE[q.dtype]
    if entry == "noalloc":
        code = attn_decode_noalloc_ptr(*ptrs, B, Hq, Hkv, Nq, Ncap, Nnew, d, scale, True, dtc,
                                       splits, stream)
    else:
        s = splits or attn_decode_num_splits(B, Hq, Hkv, Nq, Ncap, d)
        nbytes = attn_decode_workspace_size(B, Hq, Nq, d, s)
        ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")
        code = attn_decode_ptr(*ptrs[:8], ws.data_ptr(), nbytes, B, Hq, Hkv, Nq, Ncap, Nnew, d,
                               scale, True, dtc, s, stream)
    assert code == _lib.ATTN_OK, code
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu(), kc.cpu(), vc.cpu()


def compare(a, b, what):
    o_a, l_a, kc_a, vc_a = a
    o_b, l_b, kc_b, vc_b = b
    assert torch.equal(kc_a, kc_b) and torch.equal(vc_a, vc_b), what  # integer data movement
    err = (o_a.double() - o_b.double()).abs()
    assert torch.isfinite(o_a).all(), what
    assert err.max().item() <= MAX_ABS and err.mean().item() <= MEAN_ABS, (what, err.max().item())
    fin = torch.isfinite(l_b)
    assert torch.equal(torch.isfinite(l_a), fin), what
    assert torch.all(l_a[~fin] == -math.inf), what
    if fin.any():
        assert (l_a[fin] - l_b[fin]).abs().max().item() <= LSE_ABS, what
    return torch.equal(o_a, o_b) and torch.equal(l_a, l_b)


# (B, Hq, Hkv, Nq, Ncap, cache lengths, Nnew, d, dtype, splits), largest first
CASES = [
    (2, 16, 4, 4, 8192, [6000, 3000], 2, 128, "bf16", 16),
    (1, 8, 8, 1, 2048, [1500], 1, 64, "fp16", 0),
    (1, 4, 2, 2, 1024, [0], 3, 256, "bf16", 4),
]


def test_noalloc_matches_attn_decode_on_calls_in_a_row():
    bitwise = []
    for i, (B, Hq, Hkv, Nq, Ncap, lens, Nnew, d, dt, splits) in enumerate(CASES):
        print(f"[noalloc] case {i}: B{B} Hq{Hq} Hkv{Hkv} Nq{Nq} Ncap{Ncap} lens{lens} Nnew{Nnew} "
              f"d{d} {dt} splits {splits}", flush=True)
        case = make_case(B, Hq, Hkv, Nq, Ncap, lens, Nnew, d, dt, 700 + 10 * i)
        ref = run("workspace", case, B, Hq, Hkv, Nq, Ncap, Nnew, d, splits)
        got = run("noalloc", case, B, Hq, Hkv, Nq, Ncap, Nnew, d, splits)
        bitwise.append(compare(got, ref, f"case {i}"))
    # same kernels, same splits, same inputs: bitwise equal as well
    assert all(bitwise), bitwise


def test_noalloc_lowers_the_split_count_to_fit():
    # attn_decode's choice here is 32 splits (16.9 MB of partials); the
    # no-allocation call uses what fits its 8 MiB and agrees within the bar,
    # then a smaller call after it still agrees bitwise with attn_decode
    B, Hq, Hkv, Nq, Ncap, Nnew, d = 1, 64, 8, 16, 4096, 0, 128
    assert attn_decode_num_splits(B, Hq, Hkv, Nq, Ncap, d) == 32
    case = make_case(B, Hq, Hkv, Nq, Ncap, [4000], Nnew, d, "bf16", 790)
    print("[noalloc] lowered split count", flush=True)
    compare(run("noalloc", case, B, Hq, Hkv, Nq, Ncap, Nnew, d, 0),
            run("workspace", case, B, Hq, Hkv, Nq, Ncap, Nnew, d, 0), "lowered splits")
    small = make_case(1, 8, 2, 1, 512, [300], 1, 128, "bf16", 795)
    print("[noalloc] smaller call after it", flush=True)
    assert compare(run("noalloc", small, 1, 8, 2, 1, 512, 1, 128, 8),
                   run("workspace", small, 1, 8, 2, 1, 512, 1, 128, 8), "smaller after lowered")


def test_noalloc_rejects_an_explicit_count_that_does_not_fit():
    case = make_case(1, 64, 8, 16, 4096, [4000], 0, 128, "bf16", 799)
    q, kc, vc, sl, _, _ = (t.cuda() if t is not None else None for t in case)
    out = torch.empty_like(q)
    lse = torch.empty((1, 64, 16), dtype=torch.float32, device="cuda")
    code = attn_decode_noalloc_ptr(q.data_ptr(), kc.data_ptr(), vc.data_ptr(), sl.data_ptr(), 0, 0,
                                   out.data_ptr(), lse.data_ptr(), 1, 64, 8, 16, 4096, 0, 128,
                                   0.088, True, _lib.ATTN_DTYPE_BF16, 32,
                                   torch.cuda.current_stream().cuda_stream)
    assert code == _lib.ATTN_ERR_SCRATCH_LIMIT
