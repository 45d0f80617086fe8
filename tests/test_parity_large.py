"""GPU parity at the size limits: key/value tensors and KV caches whose byte
offsets pass 2^32, so that every address the kernels form in 64 bits is
exercised.  The large tensors are built on the GPU by tiling a seeded block
of rows; the oracle sees exactly the rows the attention can reach (a sliding
window in the forward, the filled cache rows in decode)."""

import math

import numpy as np
import pytest
import torch

import oracle
from attn_workloads import make_qkv

pytestmark = pytest.mark.gpu

MAX_ABS, MEAN_ABS, LSE_ABS = 1e-2, 1e-3, 1e-3


def assert_close(out, lse, O, L, what=""):
    o = out.double().numpy()
    err = np.abs(o - O)
    assert np.isfinite(o).all(), what
    assert err.max() <= MAX_ABS and err.mean() <= MEAN_ABS, (what, err.max(), err.mean())
    lg = lse.double().numpy()
    fin = np.isfinite(L)
    assert np.array_equal(np.isfinite(lg), fin), what
    if fin.any():
        assert np.abs(lg[fin] - L[fin]).max() <= LSE_ABS, what


def test_windowed_forward_reads_keys_past_4gib():
    # 18M key rows of 128 bf16 values: K and V are 4.6 GB each; a causal
    # window of 1000 keys makes every row attend only to keys near the end.
    from exact_tiled_attention_35_amd import attn_fwd

    Nq, Nk, Hq, Hkv, d, P = 300, 18_000_000, 2, 1, 128, 65536
    left = 1000
    q, ks, vs = make_qkv(1, Nq, P, Hq, Hkv, d, "bf16", 1.0, 1400)
    reps = (Nk + P - 1) // P
    kg = ks.cuda().repeat(1, reps, 1, 1)[:, :Nk]
    vg = vs.cuda().repeat(1, reps, 1, 1)[:, :Nk]
    assert kg.is_contiguous() and kg.numel() * 2 > 2**32
    scale = 1.0 / math.sqrt(d)
    out, lse = attn_fwd(q.cuda(), kg, vg, scale, True, window=(left, -1))
    torch.cuda.synchronize()
    del kg, vg
    # the last S keys hold every key any row can see; with the same
    # bottom-right alignment the sliced problem has the same visible sets
    S = Nq + left + 64
    idx = torch.arange(Nk - S, Nk) % P
    O, L = oracle.attention(q, ks[:, idx], vs[:, idx], scale, True, window=(left, -1))
    assert_close(out.cpu(), lse.cpu(), O, L, "windowed forward")


def test_decode_cache_batches_past_4gib():
    # Three sequences, each cache 2.05 GB (the per-sequence limit): the last
    # sequence starts 4.1 GB into the caches.
    from exact_tiled_attention_35_amd import attn_decode

    B, Hq, Hkv, d, Ncap, R = 3, 8, 1, 128, 8_000_000, 2048
    lens = [5, 700, 2000]
    scale = 1.0 / math.sqrt(d)
    q = make_qkv(B, 1, 1, Hq, Hq, d, "bf16", 1.0, 1410)[0]
    _, kr, vr = make_qkv(B, 1, R, 1, Hkv, d, "bf16", 1.0, 1411)
    _, kn, vn = make_qkv(B, 1, 1, 1, Hkv, d, "bf16", 1.0, 1412)
    kc = torch.zeros(B, Ncap, Hkv, d, dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    assert kc.numel() * 2 > 2**32
    kc[:, :R] = kr.cuda()
    vc[:, :R] = vr.cuda()
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    out, lse = attn_decode(q.cuda(), kc, vc, sl, kn.cuda(), vn.cuda(), scale)
    torch.cuda.synchronize()
    for b in range(B):
        n = lens[b]
        assert torch.equal(kc[b, n].cpu(), kn[b, 0]) and torch.equal(vc[b, n].cpu(), vn[b, 0]), b
        keys = torch.cat([kr[b, :n], kn[b]], 0)[None]
        vals = torch.cat([vr[b, :n], vn[b]], 0)[None]
        O, L = oracle.attention(q[b:b + 1], keys, vals, scale, True)
        assert_close(out[b:b + 1].cpu(), lse[b:b + 1].cpu(), O, L, f"decode sequence {b}")
    del kc, vc
