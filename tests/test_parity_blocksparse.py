"""GPU parity of the block-sparse forward (attn_fwd_blocksparse) against the
fp64 oracle at the forward's tolerances (max-abs 1e-2, mean-abs 1e-3, lse
1e-3; rows that keep no key exactly 0 / -inf), and bitwise against the
plain and the packed variable-length forward where they compute the same
thing with the same tiles."""

import math

import numpy as np
import pytest
import torch

import oracle
from attn_workloads import (BLOCK, BLOCKSPARSE_WORKLOADS, WORKLOADS, make_block_mask, make_qkv,
                            make_varlen, make_workload)

pytestmark = pytest.mark.gpu

MAX_ABS, MEAN_ABS, LSE_ABS = 1e-2, 1e-3, 1e-3


def gpu_bs(q, k, v, mask, scale, causal):
    from exact_tiled_attention_35_amd import attn_fwd_blocksparse

    out, lse = attn_fwd_blocksparse(q.cuda(), k.cuda(), v.cuda(), mask.cuda(), scale, causal)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


def gpu_plain(q, k, v, scale, causal):
    from exact_tiled_attention_35_amd import attn_fwd

    out, lse = attn_fwd(q.cuda(), k.cuda(), v.cuda(), scale, causal)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


def assert_close(o, lg, O, L, what=""):
    """o, O: [..., d] rows; lg, L: the matching logsumexps."""
    o, lg = np.asarray(o, dtype=np.float64), np.asarray(lg, dtype=np.float64)
    assert np.all(np.isfinite(o)), what
    err = np.abs(o - O)
    assert err.max() <= MAX_ABS, f"{what}: max-abs {err.max():.3e}"
    assert err.mean() <= MEAN_ABS, f"{what}: mean-abs {err.mean():.3e}"
    fin = np.isfinite(L)
    assert np.array_equal(np.isfinite(lg), fin), what
    assert np.all(lg[~fin] == -np.inf), what
    if fin.any():
        lerr = np.abs(lg[fin] - L[fin]).max()
        assert lerr <= LSE_ABS, f"{what}: lse max-abs {lerr:.3e}"


def nblocks(n):
    return -(-n // BLOCK)


# (B, Nq, Nk, Hq, Hkv, d, dtype, mask heads, density): several 128-row and
# 128-key blocks with ragged tails, Nq > Nk and Nq < Nk (bottom-right
# causal), MQA/GQA, every head dim, both dtypes, shared and per-head masks.
CASES = [
    (2, 300, 500, 4, 2, 128, "bf16", 4, 0.5),
    (1, 513, 257, 8, 1, 64, "fp16", 1, 0.4),
    (1, 256, 384, 2, 2, 256, "bf16", 2, 0.6),
    (2, 129, 129, 4, 4, 128, "fp16", 4, 0.3),
    (1, 400, 200, 2, 1, 128, "bf16", 1, 0.7),
    (1, 700, 1100, 4, 2, 64, "bf16", 4, 0.2),
]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("ci", range(len(CASES)))
def test_against_oracle(ci, causal):
    B, Nq, Nk, Hq, Hkv, d, dt, Hm, dens = CASES[ci]
    q, k, v = make_qkv(B, Nq, Nk, Hq, Hkv, d, dt, 1.0, 900 + ci)
    mask = make_block_mask(B, Hm, nblocks(Nq), nblocks(Nk), dens, 950 + ci)
    mask[0, 0, 0, :] = 0  # a query block that keeps no key
    if nblocks(Nq) > 1:
        mask[-1, -1, 1, :] = 0
        mask[-1, -1, 1, -1] = 1  # a block that keeps only the ragged last key block
    scale = 1.0 / math.sqrt(d)
    out, lse = gpu_bs(q, k, v, mask, scale, causal)
    O, L = oracle.attention_block_sparse(q, k, v, mask, scale, causal)
    assert_close(out.double().numpy(), lse.double().numpy(), O, L, f"case {ci} causal {causal}")
    assert (out[0, :BLOCK, 0] == 0).all() and torch.isneginf(lse[0, 0, :BLOCK]).all()


@pytest.mark.parametrize("causal", [False, True])
def test_all_ones_is_attn_fwd(causal):
    # Causal: the same tiles in the same order through the same bodies (key
    # count a multiple of 64, so that no ragged tile takes the split-P path
    # only the block-sparse instance uses when not causal; 144 blocks of 128
    # rows, so that attn_fwd runs its 128-row kernel rather than the key-split
    # one), so bit for bit.  Not causal: attn_fwd walks the keys in 128-key
    # tiles (its workgroups of 256 rows), the block-sparse call in 64-key
    # tiles (a mask block is one 128-row workgroup), so the online softmax
    # rescales at other points and the two agree to rounding: both meet the
    # parity bar against the oracle, and lse within fp32 rounding.
    B, Nq, Nk, Hq, Hkv, d = 2, 320, 448, 24, 6, 128
    q, k, v = make_qkv(B, Nq, Nk, Hq, Hkv, d, "bf16", 1.0, 971)
    mask = torch.ones((B, 1, nblocks(Nq), nblocks(Nk)), dtype=torch.uint8)
    a, la = gpu_bs(q, k, v, mask, 0.09, causal)
    b, lb = gpu_plain(q, k, v, 0.09, causal)
    if causal:
        assert torch.equal(a, b) and torch.equal(la, lb)
    else:
        O, L = oracle.attention(q, k, v, 0.09, False)
        assert_close(a.double().numpy(), la.double().numpy(), O, L, "block-sparse")
        assert_close(b.double().numpy(), lb.double().numpy(), O, L, "attn_fwd")
        assert (la - lb).abs().max().item() <= 1e-5


def test_empty_mask_gives_zero_rows():
    q, k, v = make_qkv(1, 200, 300, 4, 4, 64, "fp16", 1.0, 972)
    mask = torch.zeros((1, 4, 2, 3), dtype=torch.uint8)
    out, lse = gpu_bs(q, k, v, mask, 0.125, False)
    assert (out == 0).all() and torch.isneginf(lse).all()


@pytest.mark.parametrize("causal", [False, True])
def test_block_diagonal_documents_are_varlen(causal):
    # documents of whole blocks packed into one sequence; the mask keeps the
    # blocks of each document with itself (document masking).  Causal: bit
    # for bit the packed-sequence call; not causal: that call walks 128-key
    # tiles, this one 64-key tiles, so both are held to the oracle instead.
    docs, Hq, Hkv, d = [256, 512, 128, 384], 4, 2, 128
    q, k, v, cu_q, cu_k = make_varlen(docs, docs, Hq, Hkv, d, "bf16", 1.0, seed=973)
    N, nb = sum(docs), sum(docs) // BLOCK
    mask = torch.zeros((1, 1, nb, nb), dtype=torch.uint8)
    for s0, s1 in zip(cu_q[:-1].tolist(), cu_q[1:].tolist()):
        mask[0, 0, s0 // BLOCK:s1 // BLOCK, s0 // BLOCK:s1 // BLOCK] = 1
    out, lse = gpu_bs(q[None], k[None], v[None], mask, 0.1, causal)
    from exact_tiled_attention_35_amd import attn_fwd_varlen

    ov, lv = attn_fwd_varlen(q.cuda(), k.cuda(), v.cuda(), cu_q.cuda(), cu_k.cuda(), max(docs), 0.1,
                             causal)
    torch.cuda.synchronize()
    if causal:
        assert torch.equal(out[0], ov.cpu()) and torch.equal(lse[0], lv.cpu())
    else:
        O, L = oracle.attention_varlen(q, k, v, cu_q, cu_k, 0.1, False)
        assert_close(out[0].double().numpy(), lse[0].double().numpy(), O, L, "block-sparse")
        assert_close(ov.cpu().double().numpy(), lv.cpu().double().numpy(), O, L, "varlen")
        assert (lse[0] - lv.cpu()).abs().max().item() <= 1e-5


def test_run_to_run_bitwise_determinism():
    B, Nq, Nk, Hq, Hkv, d, dt, Hm, dens = CASES[0]
    q, k, v = make_qkv(B, Nq, Nk, Hq, Hkv, d, dt, 1.0, 974)
    mask = make_block_mask(B, Hm, nblocks(Nq), nblocks(Nk), dens, 975)
    a = gpu_bs(q, k, v, mask, 0.1, True)
    b = gpu_bs(q, k, v, mask, 0.1, True)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("name", list(BLOCKSPARSE_WORKLOADS))
def test_workload_full_size(name):
    """The benched block-sparse workloads at full size, in the launch
    configuration bench.py times; rows of three query blocks of four
    (batch, head) pairs against the oracle evaluated row by row."""
    spec = BLOCKSPARSE_WORKLOADS[name]
    w = WORKLOADS[spec["base"]]
    q, k, v = make_workload(w)
    mask = make_block_mask(w.B, w.Hq, nblocks(w.Nq), nblocks(w.Nk), spec["density"], spec["mask_seed"])
    out, lse = gpu_bs(q, k, v, mask, w.scale, w.causal)
    nqb = nblocks(w.Nq)
    for b, h in ((0, 0), (w.B - 1, w.Hq - 1), (w.B // 2, 5), (0, w.Hq // 2)):
        for qb in (0, nqb // 2, nqb - 1):
            rows = np.arange(qb * BLOCK, min(w.Nq, qb * BLOCK + BLOCK))
            O, L = oracle.attention_block_sparse_rows(q, k, v, mask, w.scale, w.causal, b, h, rows)
            assert_close(out[b, rows, h].double().numpy(), lse[b, h, rows].double().numpy(), O, L,
                         f"{name} b{b} h{h} block {qb}")
