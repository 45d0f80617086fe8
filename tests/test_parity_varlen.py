"""GPU parity of the packed variable-length forward (attn_fwd_varlen)
against the fp64 oracle, at the forward's tolerances (max-abs 1e-2,
mean-abs 1e-3, lse 1e-3; rows with no visible key exactly 0 / -inf), and
bitwise against the batched forward where both compute the same thing."""

import math

import numpy as np
import pytest
import torch

import oracle
from attn_workloads import VARLEN_WORKLOADS, make_qkv, make_varlen, varlen_lengths

pytestmark = pytest.mark.gpu

MAX_ABS, MEAN_ABS, LSE_ABS = 1e-2, 1e-3, 1e-3


def gpu_varlen(q, k, v, cu_q, cu_k, max_q, scale, causal):
    from exact_tiled_attention_35_amd import attn_fwd_varlen

    out, lse = attn_fwd_varlen(q.cuda(), k.cuda(), v.cuda(), cu_q.cuda(), cu_k.cuda(), max_q,
                               scale, causal)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


def gpu_batched(q, k, v, scale, causal):
    from exact_tiled_attention_35_amd import attn_fwd

    out, lse = attn_fwd(q.cuda(), k.cuda(), v.cuda(), scale, causal)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


def assert_close(out, lse, O, L, what=""):
    o = out.double().numpy()
    lg = lse.double().numpy()
    err = np.abs(o - O)
    assert np.all(np.isfinite(o)), what
    if err.size:
        assert err.max() <= MAX_ABS, f"{what}: max-abs {err.max():.3e}"
        assert err.mean() <= MEAN_ABS, f"{what}: mean-abs {err.mean():.3e}"
    fin = np.isfinite(L)
    assert np.array_equal(np.isfinite(lg), fin), what
    assert np.all(lg[~fin] == -np.inf), what
    if o.ndim == 3:  # packed [total_q, Hq, d] against lse [Hq, total_q]
        assert np.all(o[~fin.T] == 0.0), what
    if fin.any():
        lerr = np.abs(lg[fin] - L[fin]).max()
        assert lerr <= LSE_ABS, f"{what}: lse max-abs {lerr:.3e}"


# (lens_q, lens_k, Hq, Hkv, d, dtype): ragged sequences spanning several
# 128-row and 64-key tiles with ragged tails; empty query sequences, a
# sequence with queries but no keys, single rows, Nq > Nk and Nq < Nk per
# sequence (bottom-right causal), MQA/GQA, every head dim, both dtypes.
CASES = [
    ([1, 200, 0, 513, 64, 130], None, 8, 2, 128, "bf16"),
    ([100, 7, 300, 0, 65], [300, 0, 129, 50, 1], 4, 4, 64, "fp16"),
    ([257, 31, 128], [257, 400, 1], 4, 1, 256, "bf16"),
    ([129, 1, 1, 700], [64, 1000, 2, 700], 6, 3, 128, "fp16"),
    ([5, 0, 0, 3], [0, 4, 0, 9], 2, 1, 64, "bf16"),
]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("ci", range(len(CASES)))
def test_ragged_against_oracle(ci, causal):
    lens_q, lens_k, Hq, Hkv, d, dt = CASES[ci]
    lens_k = lens_k or lens_q
    q, k, v, cu_q, cu_k = make_varlen(lens_q, lens_k, Hq, Hkv, d, dt, 1.0, 500 + ci)
    scale = 1.0 / math.sqrt(d)
    out, lse = gpu_varlen(q, k, v, cu_q, cu_k, max(lens_q), scale, causal)
    O, L = oracle.attention_varlen(q, k, v, cu_q, cu_k, scale, causal)
    assert_close(out, lse, O, L, f"case {ci} causal {causal}")


@pytest.mark.parametrize("causal", [False, True])
def test_each_sequence_is_bitwise_the_batched_forward(causal):
    # The varlen kernel is the batched kernel with per-sequence row offsets:
    # every sequence must equal attn_fwd run on that sequence alone, bit for
    # bit.  (128 heads: even a one-row sequence has the 128 row blocks above
    # which attn_fwd runs its 128-row kernel rather than the key-split one.)
    lens_q, lens_k = [129, 1, 1, 700], [64, 1000, 2, 700]
    q, k, v, cu_q, cu_k = make_varlen(lens_q, lens_k, 128, 32, 128, "bf16", 1.0, 510)
    scale = 1.0 / math.sqrt(128)
    out, lse = gpu_varlen(q, k, v, cu_q, cu_k, max(lens_q), scale, causal)
    for b in range(len(lens_q)):
        qs, qe, ks, ke = int(cu_q[b]), int(cu_q[b + 1]), int(cu_k[b]), int(cu_k[b + 1])
        ob, lb = gpu_batched(q[None, qs:qe], k[None, ks:ke], v[None, ks:ke], scale, causal)
        assert torch.equal(out[qs:qe], ob[0]), b
        assert torch.equal(lse[:, qs:qe], lb[0]), b


@pytest.mark.parametrize("causal", [False, True])
def test_equal_lengths_are_bitwise_the_padded_batch(causal):
    B, N, Hq, Hkv, d = 3, 300, 16, 2, 64  # 144 row blocks: attn_fwd's 128-row kernel
    q, k, v = make_qkv(B, N, N, Hq, Hkv, d, "fp16", 1.0, 511)
    cu = torch.arange(0, (B + 1) * N, N, dtype=torch.int32)
    out, lse = gpu_varlen(q.reshape(B * N, Hq, d), k.reshape(B * N, Hkv, d),
                          v.reshape(B * N, Hkv, d), cu, cu, N, 0.125, causal)
    ob, lb = gpu_batched(q, k, v, 0.125, causal)
    assert torch.equal(out, ob.reshape(B * N, Hq, d))
    assert torch.equal(lse, lb.transpose(0, 1).reshape(Hq, B * N))


def test_no_keys_at_all():
    # total_k = 0: k and v are empty (NULL); every row gives 0 / -inf.
    q, _, _, cu_q, _ = make_varlen([3, 70], [0, 0], 4, 2, 128, "bf16", 1.0, 512)
    k = torch.empty(0, 2, 128, dtype=torch.bfloat16)
    cu_k = torch.zeros(3, dtype=torch.int32)
    out, lse = gpu_varlen(q, k, k, cu_q, cu_k, 70, 0.1, False)
    assert torch.equal(out, torch.zeros_like(out))
    assert torch.isneginf(lse).all()


def test_out_of_range_prefix_sums_are_clamped():
    # cu_seqlens beyond [0, total] are clamped, and a decreasing pair is an
    # empty sequence (the documented reading of malformed prefix sums).
    q, k, v, _, _ = make_varlen([40, 60], [50, 50], 2, 2, 64, "bf16", 1.0, 513)
    cu_q = torch.tensor([0, 40, 10 ** 6], dtype=torch.int32)
    cu_k = torch.tensor([-5, 50, 10 ** 6], dtype=torch.int32)
    out, lse = gpu_varlen(q, k, v, cu_q, cu_k, 128, 0.125, True)
    O, L = oracle.attention_varlen(q, k, v, [0, 40, 100], [0, 50, 100], 0.125, True)
    assert_close(out, lse, O, L)
    # a decreasing pair: sequence 1 has no query rows, sequence 2 starts at 30
    cu_q = torch.tensor([0, 40, 30, 100], dtype=torch.int32)
    cu_k = torch.tensor([0, 50, 60, 100], dtype=torch.int32)
    out2, lse2 = gpu_varlen(q, k, v, cu_q, cu_k, 128, 0.125, False)
    O2, L2 = oracle.attention_varlen(q, k, v, [0, 40, 40, 100], [0, 50, 60, 100], 0.125, False)
    # rows 30..39 belong to sequence 0 and to the clamped sequence 2 alike;
    # only rows owned by exactly one sequence are compared
    assert_close(out2[40:], lse2[:, 40:], O2[40:], L2[:, 40:])


def test_run_to_run_bitwise_determinism():
    q, k, v, cu_q, cu_k = make_varlen([300, 5, 777], [300, 900, 777], 8, 2, 128, "bf16", 1.0, 514)
    a = gpu_varlen(q, k, v, cu_q, cu_k, 777, 0.088, True)
    b = gpu_varlen(q, k, v, cu_q, cu_k, 777, 0.088, True)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("name", list(VARLEN_WORKLOADS))
def test_packed_workload_full_size(name):
    # 16384 packed tokens in sequences of 256..4096, 16 heads of 128: the
    # launch the bench times; sampled rows of several sequences against the
    # oracle, every row against the convex-combination bound.
    wl = VARLEN_WORKLOADS[name]
    causal = wl["causal"]
    lens = varlen_lengths(wl["total"], wl["lo"], wl["hi"], wl["seed"])
    print(f"[parity] {wl['name']} causal={causal} lens={lens}", flush=True)
    q, k, v, cu_q, cu_k = make_varlen(lens, lens, wl["H"], wl["H"], wl["d"], wl["dtype"], 1.0,
                                      wl["seed"])
    scale = 1.0 / math.sqrt(wl["d"])
    out, lse = gpu_varlen(q, k, v, cu_q, cu_k, max(lens), scale, causal)
    assert torch.isfinite(out).all() and torch.isfinite(lse).all()
    rng = np.random.default_rng(wl["seed"])
    for b in sorted({0, len(lens) // 2, len(lens) - 1}):
        s, e = int(cu_q[b]), int(cu_q[b + 1])
        n = e - s
        rows = sorted({0, 1, 127, 128, n // 2, n - 1} | {int(x) for x in rng.integers(0, n, 12)})
        for h in (0, wl["H"] - 1):
            O, L = oracle.attention_rows(q[None, s:e], k[None, s:e], v[None, s:e], scale, causal,
                                         0, h, rows)
            assert_close(out[s:e][rows, h], lse[h, s:e][rows], O, L, f"seq {b} head {h}")
    # every row: within the range of the V rows it may see
    for b in range(len(lens)):
        s, e = int(cu_q[b]), int(cu_q[b + 1])
        vf = v[s:e].float()
        if causal:
            vmax, vmin = torch.cummax(vf, 0).values, torch.cummin(vf, 0).values
        else:
            vmax, vmin = vf.amax(0, keepdim=True), vf.amin(0, keepdim=True)
        of = out[s:e].float()
        assert torch.all(of <= vmax + 1e-2) and torch.all(of >= vmin - 1e-2), b
