"""GPU parity of the packed variable-length backward (attn_bwd_varlen)
against the fp64 oracle (attention_backward_varlen) with the backward's
criterion (max and mean error at most twice those of the plain
low-precision backward given the same inputs, sequence by sequence), and
bitwise against attn_bwd run on each sequence alone."""

import numpy as np
import pytest
import torch

import oracle
from attn_workloads import VARLEN_WORKLOADS, make_varlen, varlen_lengths
from test_parity_bwd import check_grads, lowp_backward

pytestmark = pytest.mark.gpu


def gpu_fwd_bwd(q, k, v, do, cu_q, cu_k, max_q, max_k, scale, causal):
    from exact_tiled_attention_35_amd import attn_bwd_varlen, attn_fwd_varlen

    qc, kc, vc, dc, cq, ck = (x.cuda() for x in (q, k, v, do, cu_q, cu_k))
    out, lse = attn_fwd_varlen(qc, kc, vc, cq, ck, max_q, scale, causal)
    dq, dk, dv, delta = attn_bwd_varlen(qc, kc, vc, out, dc, lse, cq, ck, max_q, max_k, scale, causal)
    torch.cuda.synchronize()
    return [x.cpu() for x in (dq, dk, dv, delta, out, lse)]


def lowp_varlen(q, k, v, do, out, cu_q, cu_k, scale, causal):
    dq, dk, dv = (np.zeros(x.shape) for x in (q, k, v))
    for b in range(len(cu_q) - 1):
        qs, qe, ks, ke = int(cu_q[b]), int(cu_q[b + 1]), int(cu_k[b]), int(cu_k[b + 1])
        if qe == qs or ke == ks:
            continue
        g = lowp_backward(q[None, qs:qe], k[None, ks:ke], v[None, ks:ke], do[None, qs:qe],
                          out[None, qs:qe], scale, causal)
        dq[qs:qe], dk[ks:ke], dv[ks:ke] = g[0][0], g[1][0], g[2][0]
    return dq, dk, dv


# (lens_q, lens_k, Hq, Hkv, d, dtype): several 128-row / 32-key tiles with
# ragged tails, sequences without query rows, without keys, single rows,
# Nq > Nk and Nq < Nk per sequence, MQA/GQA, every head dim, both dtypes.
CASES = [
    ([1, 200, 0, 300, 64, 130], None, 4, 2, 128, "bf16"),
    ([100, 7, 300, 0, 65], [300, 0, 129, 50, 1], 4, 4, 64, "fp16"),
    ([257, 31, 128], [257, 400, 1], 2, 1, 256, "bf16"),
    ([129, 1, 1, 400], [64, 500, 2, 400], 6, 3, 128, "fp16"),
]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("ci", range(len(CASES)))
def test_varlen_backward_against_oracle(ci, causal):
    lens_q, lens_k, Hq, Hkv, d, dt = CASES[ci]
    lens_k = lens_k or lens_q
    q, k, v, cu_q, cu_k = make_varlen(lens_q, lens_k, Hq, Hkv, d, dt, 1.0, 1300 + ci)
    do = make_varlen(lens_q, lens_k, Hq, Hkv, d, dt, 1.0, 1350 + ci)[0]
    scale = 1.0 / np.sqrt(d)
    dq, dk, dv, delta, out, lse = gpu_fwd_bwd(q, k, v, do, cu_q, cu_k, max(lens_q), max(lens_k),
                                              scale, causal)
    want = oracle.attention_backward_varlen(q, k, v, do, cu_q, cu_k, scale, causal)
    base = lowp_varlen(q, k, v, do, out, cu_q, cu_k, scale, causal)
    check_grads((dq, dk, dv), want[:3], base, f"case {ci} causal {causal}")
    # delta = sum(dout * out) from the rounded out, within its rounding bound
    ulp = 2.0 ** -7 if dt == "bf16" else 2.0 ** -10
    bound = (np.abs(do.double().numpy()) * (np.abs(out.double().numpy()) * ulp + 1e-5)).sum(-1).T + 1e-5
    assert np.all(np.abs(delta.double().numpy() - want[3]) <= bound)
    # keys of sequences without query rows and query rows without keys: zero
    for b in range(len(lens_q)):
        qs, qe = int(cu_q[b]), int(cu_q[b + 1])
        ks, ke = int(cu_k[b]), int(cu_k[b + 1])
        if qe == qs:
            assert (dk[ks:ke] == 0).all() and (dv[ks:ke] == 0).all()
        if ke == ks:
            assert (dq[qs:qe] == 0).all()


@pytest.mark.parametrize("causal", [False, True])
def test_each_sequence_is_bitwise_attn_bwd(causal):
    from exact_tiled_attention_35_amd import attn_bwd

    lens_q, lens_k, Hq, Hkv, d = [300, 129, 64], [200, 129, 500], 4, 2, 128
    q, k, v, cu_q, cu_k = make_varlen(lens_q, lens_k, Hq, Hkv, d, "bf16", 1.0, 1390)
    do = make_varlen(lens_q, lens_k, Hq, Hkv, d, "bf16", 1.0, 1391)[0]
    dq, dk, dv, delta, outv, lsev = gpu_fwd_bwd(q, k, v, do, cu_q, cu_k, max(lens_q), max(lens_k),
                                                0.1, causal)
    for b in range(len(lens_q)):
        qs, qe, ks, ke = int(cu_q[b]), int(cu_q[b + 1]), int(cu_k[b]), int(cu_k[b + 1])
        qc, dc = q[None, qs:qe].cuda(), do[None, qs:qe].cuda()
        kc, vc = k[None, ks:ke].cuda(), v[None, ks:ke].cuda()
        # the backward of each sequence alone, from the same forward output
        # (a sequence's own attn_fwd may take the key-split kernel for its
        # small grid, whose output differs in rounding order)
        out = outv[None, qs:qe].contiguous().cuda()
        lse = lsev[None, :, qs:qe].contiguous().cuda()
        g = [x.cpu() for x in attn_bwd(qc, kc, vc, out, dc, lse, 0.1, causal)]
        torch.cuda.synchronize()
        assert torch.equal(dq[qs:qe], g[0][0]) and torch.equal(dk[ks:ke], g[1][0])
        assert torch.equal(dv[ks:ke], g[2][0]) and torch.equal(delta[:, qs:qe], g[3][0])


def test_varlen_backward_is_deterministic():
    lens_q, lens_k, Hq, Hkv, d, dt = CASES[3]
    q, k, v, cu_q, cu_k = make_varlen(lens_q, lens_k, Hq, Hkv, d, dt, 1.0, 1392)
    do = make_varlen(lens_q, lens_k, Hq, Hkv, d, dt, 1.0, 1393)[0]
    a = gpu_fwd_bwd(q, k, v, do, cu_q, cu_k, max(lens_q), max(lens_k), 0.1, True)
    b = gpu_fwd_bwd(q, k, v, do, cu_q, cu_k, max(lens_q), max(lens_k), 0.1, True)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_packed_workload_full_size_sequences():
    """The causal packed workload (16,384 tokens, 16 heads, d 128) at full
    size; two sequences' gradients against the oracle."""
    wl = VARLEN_WORKLOADS["varlen_causal_t16384_len256to4096_h16_d128_bf16"]
    lens = varlen_lengths(wl["total"], wl["lo"], wl["hi"], wl["seed"])
    H, d = wl["H"], wl["d"]
    q, k, v, cu_q, cu_k = make_varlen(lens, lens, H, H, d, wl["dtype"], 1.0, wl["seed"])
    do = make_varlen(lens, lens, H, H, d, wl["dtype"], 1.0, wl["seed"] + 100)[0]
    scale = float(np.float32(1.0 / np.sqrt(d)))
    dq, dk, dv, delta, out, lse = gpu_fwd_bwd(q, k, v, do, cu_q, cu_k, max(lens), max(lens), scale, True)
    for b in (1, len(lens) - 1):  # a short and a longer sequence
        s0, s1 = int(cu_q[b]), int(cu_q[b + 1])
        sl = slice(s0, s1)
        want = oracle.attention_backward(q[None, sl], k[None, sl], v[None, sl], do[None, sl], scale, True)
        base = lowp_backward(q[None, sl], k[None, sl], v[None, sl], do[None, sl], out[None, sl], scale, True)
        check_grads((dq[None, sl], dk[None, sl], dv[None, sl]), want[:3], base, f"sequence {b}")
