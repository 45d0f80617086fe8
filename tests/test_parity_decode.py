"""GPU parity of the KV-cache decode forward (attn_decode) against the fp64
oracle.

The cache append is integer data movement, so the updated caches must match
bit for bit.  The attention of batch b is the oracle's forward on the query
rows of b against the first cache_seqlens[b] + Nnew rows of b's updated
cache, with the forward's tolerances (max-abs 1e-2, mean-abs 1e-3, lse
1e-3, rows without keys exactly 0 / -inf).
"""

import math

import numpy as np
import pytest
import torch

import oracle
from attn_workloads import make_qkv

pytestmark = pytest.mark.gpu

MAX_ABS, MEAN_ABS, LSE_ABS = 1e-2, 1e-3, 1e-3


def run_case(B, Hq, Hkv, Nq, Ncap, Nnew, d, dt, causal, lens, splits, seed, scale=None):
    from exact_tiled_attention_35_amd import attn_decode

    q = make_qkv(B, Nq, Nq, Hq, Hq, d, dt, 1.0, seed)[0]
    _, kc, vc = make_qkv(B, 1, Ncap, 1, Hkv, d, dt, 1.0, seed + 1)
    _, kn, vn = make_qkv(B, 1, max(Nnew, 1), 1, Hkv, d, dt, 1.0, seed + 2)
    kn, vn = kn[:, :Nnew].contiguous(), vn[:, :Nnew].contiguous()
    seqlens = torch.tensor(lens, dtype=torch.int32)
    # expected caches after the append (rows at or past Ncap are not written)
    ke, ve = kc.clone(), vc.clone()
    for b in range(B):
        m = max(0, min(Nnew, Ncap - lens[b]))
        ke[b, lens[b]:lens[b] + m] = kn[b, :m]
        ve[b, lens[b]:lens[b] + m] = vn[b, :m]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    kg, vg = kc.cuda(), vc.cuda()
    out, lse = attn_decode(q.cuda(), kg, vg, seqlens.cuda(), kn.cuda() if Nnew else None,
                           vn.cuda() if Nnew else None, scale, causal, splits)
    torch.cuda.synchronize()
    assert torch.equal(kg.cpu(), ke) and torch.equal(vg.cpu(), ve), "cache append"
    out, lse = out.cpu().double().numpy(), lse.cpu().double().numpy()
    worst = 0.0
    for b in range(B):
        n = min(Ncap, lens[b] + Nnew)
        O, L = oracle.attention(q[b:b + 1], ke[b:b + 1, :n], ve[b:b + 1, :n], scale, causal)
        err = np.abs(out[b:b + 1] - O)
        assert err.max() <= MAX_ABS and err.mean() <= MEAN_ABS, (b, err.max(), err.mean())
        fin = np.isfinite(L)
        assert np.array_equal(np.isfinite(lse[b:b + 1]), fin)
        assert np.all(lse[b:b + 1][~fin] == -np.inf) and np.all(out[b:b + 1][np.broadcast_to(
            ~fin.transpose(0, 2, 1)[..., None], out[b:b + 1].shape)] == 0)
        if fin.any():
            assert np.abs(lse[b:b + 1][fin] - L[fin]).max() <= LSE_ABS
        worst = max(worst, float(err.max()))
    return worst


CASES = [  # B, Hq, Hkv, Nq, Ncap, Nnew, d, dtype, causal, lens, splits
    (1, 1, 1, 1, 64, 1, 128, "bf16", True, [0], 1),
    (2, 8, 2, 1, 300, 1, 128, "bf16", True, [17, 250], 0),
    (3, 32, 8, 1, 1000, 1, 128, "bf16", True, [999, 0, 511], 0),
    (2, 16, 16, 4, 700, 4, 128, "fp16", True, [96, 500], 3),
    (2, 8, 1, 16, 600, 16, 64, "bf16", True, [0, 584], 5),
    (1, 8, 2, 7, 2048, 7, 256, "fp16", False, [1500], 0),
    (4, 4, 4, 2, 257, 0, 128, "bf16", False, [257, 0, 100, 33], 2),   # no append; one row set empty
    (2, 64, 8, 1, 4096, 1, 128, "bf16", True, [4095, 1000], 16),
    (1, 32, 4, 16, 513, 16, 128, "bf16", True, [200], 0),              # 128 packed rows per KV head
    (1, 40, 4, 16, 300, 2, 64, "bf16", True, [40], 4),                 # 160 packed rows: two row blocks
    (2, 8, 2, 2, 700, 40, 64, "fp16", True, [20, 600], 5),             # new rows across tiles and splits
    (1, 8, 2, 3, 300, 16, 128, "bf16", True, [290], 3),                # new rows past Ncap are dropped
    (1, 48, 4, 12, 400, 12, 128, "bf16", True, [100], 4),              # two row blocks append once
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B%dH%d-%dq%dcap%dnew%dd%d%s%s-s%d" % (
    c[0], c[1], c[2], c[3], c[4], c[5], c[6], c[7], "c" if c[8] else "", c[10]))
def test_decode_against_oracle(case):
    w = run_case(*case, seed=800 + CASES.index(case))
    print(f"[parity-decode] {case}: max-abs {w:.3e}", flush=True)


def test_decode_splits_agree_with_one_split():
    # The logsumexp merge of key ranges reproduces the one-range result up to
    # fp32 rounding of the partial outputs.
    from exact_tiled_attention_35_amd import attn_decode

    q = make_qkv(2, 1, 1, 16, 16, 128, "bf16", 1.0, 900)[0].cuda()
    _, kc, vc = make_qkv(2, 1, 3000, 1, 4, 128, "bf16", 1.0, 901)
    sl = torch.tensor([2999, 1234], dtype=torch.int32).cuda()
    ref = attn_decode(q, kc.cuda(), vc.cuda(), sl, None, None, None, True, 1)
    for s in (2, 7, 64):
        got = attn_decode(q, kc.cuda(), vc.cuda(), sl, None, None, None, True, s)
        assert (got[0].double() - ref[0].double()).abs().max() <= 8e-3
        assert (got[1] - ref[1]).abs().max() <= 1e-5


def test_decode_matches_forward_when_cache_is_full():
    # Nq rows against a full cache equals attn_fwd on the same tensors.
    from exact_tiled_attention_35_amd import attn_decode, attn_fwd

    q = make_qkv(2, 8, 8, 8, 8, 128, "bf16", 1.0, 902)[0].cuda()
    _, k, v = make_qkv(2, 1, 512, 1, 2, 128, "bf16", 1.0, 903)
    k, v = k.cuda(), v.cuda()
    sl = torch.full((2,), 512, dtype=torch.int32).cuda()
    o1, l1 = attn_decode(q, k, v, sl, None, None, None, True, 1)
    o2, l2 = attn_fwd(q, k, v, None, True)
    assert (o1.double() - o2.double()).abs().max() <= 1.6e-2
    assert (l1 - l2).abs().max() <= 1e-4


@pytest.mark.parametrize("name", ["decode_b16_hq32_hkv8_cache32768_d128_bf16",
                                  "decode_b1_hq32_hkv8_cache131072_d128_bf16"])
def test_decode_workload_full_size(name):
    # The benchmark's decode workloads, in the launch configuration bench.py
    # times (library-chosen splits), checked on every query head of a few
    # sequences against the oracle.
    from attn_workloads import DECODE_WORKLOADS
    from exact_tiled_attention_35_amd import attn_decode

    w = DECODE_WORKLOADS[name]
    q = make_qkv(w.B, w.Nq, w.Nq, w.Hq, w.Hq, w.d, w.dtype, w.sigma, w.seed)[0]
    _, kc, vc = make_qkv(w.B, 1, w.Nk, 1, w.Hkv, w.d, w.dtype, w.sigma, w.seed + 1)
    _, kn, vn = make_qkv(w.B, 1, 1, 1, w.Hkv, w.d, w.dtype, w.sigma, w.seed + 2)
    sl = torch.full((w.B,), w.Nk - 1, dtype=torch.int32)
    kg, vg = kc.cuda(), vc.cuda()
    out, lse = attn_decode(q.cuda(), kg, vg, sl.cuda(), kn.cuda(), vn.cuda(), w.scale, w.causal, 0)
    torch.cuda.synchronize()
    out, lse = out.cpu().double().numpy(), lse.cpu().double().numpy()
    kc[:, w.Nk - 1] = kn[:, 0]
    vc[:, w.Nk - 1] = vn[:, 0]
    assert torch.equal(kg[:, w.Nk - 1].cpu(), kn[:, 0]) and torch.equal(vg[:, w.Nk - 1].cpu(), vn[:, 0])
    worst = 0.0
    for b in sorted({0, w.B // 2, w.B - 1}):
        O, L = oracle.attention(q[b:b + 1], kc[b:b + 1], vc[b:b + 1], w.scale, w.causal)
        err = np.abs(out[b:b + 1] - O)
        assert err.max() <= MAX_ABS and err.mean() <= MEAN_ABS
        assert np.abs(lse[b:b + 1] - L).max() <= LSE_ABS
        worst = max(worst, float(err.max()))
    print(f"[parity-decode] {name}: worst max-abs {worst:.3e}", flush=True)


def test_decode_append_only_without_query_rows():
    # Nq = 0: the call only appends (the append kernel); with query rows the
    # attention kernel appends, and both leave the same caches.
    from exact_tiled_attention_35_amd import attn_decode

    B, Hkv, Ncap, Nnew, d = 2, 4, 200, 5, 128
    _, kc, vc = make_qkv(B, 1, Ncap, 1, Hkv, d, "bf16", 1.0, 950)
    _, kn, vn = make_qkv(B, 1, Nnew, 1, Hkv, d, "bf16", 1.0, 951)
    lens = [10, 197]  # the second sequence's last two new rows fall past Ncap
    sl = torch.tensor(lens, dtype=torch.int32).cuda()
    caches = []
    for Nq in (0, 1):
        q = make_qkv(B, max(Nq, 1), 1, 8, 8, d, "bf16", 1.0, 952)[0][:, :Nq].contiguous()
        kg, vg = kc.cuda(), vc.cuda()
        attn_decode(q.cuda(), kg, vg, sl, kn.cuda(), vn.cuda(), None, True)
        torch.cuda.synchronize()
        caches.append((kg.cpu(), vg.cpu()))
    ke, ve = kc.clone(), vc.clone()
    for b in range(B):
        m = max(0, min(Nnew, Ncap - lens[b]))
        ke[b, lens[b]:lens[b] + m] = kn[b, :m]
        ve[b, lens[b]:lens[b] + m] = vn[b, :m]
    for kg, vg in caches:
        assert torch.equal(kg, ke) and torch.equal(vg, ve)
