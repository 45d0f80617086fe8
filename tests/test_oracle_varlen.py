"""Pins of the oracle's packed variable-length attention (CPU only).

Each sequence of the packed batch is checked against the pure-Python brute
force run on that sequence alone, and an equal-length packing against the
batched oracle; planted mistakes in the packing (key offsets taken from the
query prefix sums, sequences shifted by one row) must fail the pin."""

import math

import numpy as np
import pytest

import oracle
from attn_workloads import make_varlen
from _bruteforce import brute_attention

# (lens_q, lens_k, Hq, Hkv, d, causal): empty query sequences, a sequence
# without keys, single rows, Nq != Nk per sequence (bottom-right causal).
CASES = [
    ([3, 0, 5, 1], [3, 2, 5, 4], 2, 1, 4, False),
    ([3, 0, 5, 1], [3, 2, 5, 4], 2, 1, 4, True),
    ([4, 2, 6], [2, 0, 7], 4, 2, 3, True),
    ([1, 1, 1], [5, 1, 3], 2, 2, 5, False),
]


def as_lists(x):
    return x.double().tolist()


def brute_varlen(q, k, v, cu_q, cu_k, scale, causal):
    total_q, Hq, d = q.shape
    O = np.zeros((total_q, Hq, d))
    L = np.full((Hq, total_q), -np.inf)
    for b in range(len(cu_q) - 1):
        qs, qe, ks, ke = int(cu_q[b]), int(cu_q[b + 1]), int(cu_k[b]), int(cu_k[b + 1])
        if qe == qs or ke == ks:
            continue
        Ob, Lb = brute_attention([as_lists(q[qs:qe])], [as_lists(k[ks:ke])], [as_lists(v[ks:ke])],
                                 scale, causal)
        O[qs:qe] = np.array(Ob[0])
        L[:, qs:qe] = np.array(Lb[0])
    return O, L


@pytest.mark.parametrize("case", CASES)
def test_varlen_matches_bruteforce_per_sequence(case):
    lens_q, lens_k, Hq, Hkv, d, causal = case
    q, k, v, cu_q, cu_k = make_varlen(lens_q, lens_k, Hq, Hkv, d, "bf16", 1.0, seed=11)
    scale = float(np.float32(1 / math.sqrt(d)))  # the fp32 value the library receives
    O, L = oracle.attention_varlen(q, k, v, cu_q, cu_k, scale, causal)
    Ob, Lb = brute_varlen(q, k, v, cu_q, cu_k, scale, causal)
    np.testing.assert_allclose(O, Ob, rtol=0, atol=1e-12)
    fin = np.isfinite(Lb)
    assert (np.isfinite(L) == fin).all()
    np.testing.assert_allclose(L[fin], Lb[fin], rtol=0, atol=1e-12)


def test_sequence_without_keys_gives_zero_rows():
    q, k, v, cu_q, cu_k = make_varlen([2, 3], [4, 0], 2, 2, 4, seed=3)
    O, L = oracle.attention_varlen(q, k, v, cu_q, cu_k, 0.5, False)
    assert (O[2:] == 0).all() and np.isneginf(L[:, 2:]).all()
    assert np.isfinite(L[:, :2]).all()


def test_equal_lengths_match_the_batched_oracle():
    B, N, Hq, Hkv, d = 3, 5, 4, 2, 8
    q, k, v, cu_q, cu_k = make_varlen([N] * B, [N] * B, Hq, Hkv, d, seed=5)
    for causal in (False, True):
        O, L = oracle.attention_varlen(q, k, v, cu_q, cu_k, 0.3, causal)
        Ob, Lb = oracle.attention(q.reshape(B, N, Hq, d), k.reshape(B, N, Hkv, d),
                                  v.reshape(B, N, Hkv, d), 0.3, causal)
        np.testing.assert_allclose(O, Ob.reshape(B * N, Hq, d), rtol=0, atol=1e-14)
        np.testing.assert_allclose(L, Lb.transpose(1, 0, 2).reshape(Hq, B * N), rtol=0, atol=1e-14)


@pytest.mark.parametrize("mistake", ["keys_at_query_offsets", "shifted_by_one"])
def test_planted_packing_mistakes_fail_the_pin(mistake):
    lens_q, lens_k, Hq, Hkv, d, causal = CASES[2]
    q, k, v, cu_q, cu_k = make_varlen(lens_q, lens_k, Hq, Hkv, d, "bf16", 1.0, seed=11)
    scale = float(np.float32(1 / math.sqrt(d)))  # the fp32 value the library receives
    Ob, _ = brute_varlen(q, k, v, cu_q, cu_k, scale, causal)
    if mistake == "keys_at_query_offsets":
        bad_q, bad_k = cu_q, cu_q.clamp(max=int(cu_k[-1]))
    else:
        bad_q, bad_k = cu_q, (cu_k + 1).clamp(max=int(cu_k[-1]))
        bad_k[0] = 0
    O, _ = oracle.attention_varlen(q, k, v, bad_q, bad_k, scale, causal)
    assert np.abs(O - Ob).max() > 1e-3


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_is_document_masked_attention(causal):
    # Documents packed into one sequence, each token attending only to the
    # tokens of its own document (document masking): the same as the packed
    # variable-length attention with the document boundaries as prefix sums.
    # Reference: one dense softmax over the whole packed sequence with a
    # block-diagonal mask, written out here in fp64.
    lens = [5, 1, 7, 3]
    q, k, v, cu, _ = make_varlen(lens, lens, 2, 1, 8, "bf16", 1.0, seed=21)
    scale = float(np.float32(0.35))
    O, L = oracle.attention_varlen(q, k, v, cu, cu, scale, causal)
    doc = np.repeat(np.arange(len(lens)), lens)
    T = len(doc)
    pos = np.concatenate([np.arange(n) for n in lens])
    allowed = doc[:, None] == doc[None, :]
    if causal:
        allowed &= pos[None, :] <= pos[:, None]
    qd, kd, vd = q.double().numpy(), k.double().numpy(), v.double().numpy()
    for h in range(2):
        sc = qd[:, h, :] @ kd[:, 0, :].T * scale
        sc = np.where(allowed, sc, -np.inf)
        mx = sc.max(axis=1, keepdims=True)
        w = np.exp(sc - mx)
        ref = (w / w.sum(axis=1, keepdims=True)) @ vd[:, 0, :]
        np.testing.assert_allclose(O[:, h, :], ref, rtol=0, atol=1e-12)
        np.testing.assert_allclose(L[h], (mx[:, 0] + np.log(w.sum(axis=1))), rtol=0, atol=1e-12)
    assert T == int(cu[-1])


# ---------------------------------------------------------------------------
# Gradients over packed sequences (attention_backward_varlen)
# ---------------------------------------------------------------------------
def varlen_loss(q, k, v, do, cu_q, cu_k, scale, causal):
    O, _ = oracle.attention_varlen(q, k, v, cu_q, cu_k, scale, causal)
    return float((O * do).sum())


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_gradients_match_finite_differences(causal):
    # sequences with and without query rows / keys, Nq != Nk per sequence
    lens_q, lens_k = [2, 0, 3, 1], [3, 2, 2, 0]
    rng = np.random.default_rng(101)
    tq, tk, Hq, Hkv, d = sum(lens_q), sum(lens_k), 2, 1, 2
    q, do = rng.standard_normal((tq, Hq, d)), rng.standard_normal((tq, Hq, d))
    k, v = rng.standard_normal((tk, Hkv, d)), rng.standard_normal((tk, Hkv, d))
    cu_q, cu_k = np.cumsum([0] + lens_q), np.cumsum([0] + lens_k)
    dq, dk, dv, _ = oracle.attention_backward_varlen(q, k, v, do, cu_q, cu_k, 0.8, causal)
    eps = 1e-6
    for x, g in ((q, dq), (k, dk), (v, dv)):
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            x0 = x[idx]
            x[idx] = x0 + eps
            lp = varlen_loss(q, k, v, do, cu_q, cu_k, float(np.float32(0.8)), causal)
            x[idx] = x0 - eps
            lm = varlen_loss(q, k, v, do, cu_q, cu_k, float(np.float32(0.8)), causal)
            x[idx] = x0
            fd[idx] = (lp - lm) / (2 * eps)
        assert np.abs(g - fd).max() <= 1e-7
    # the sequence without keys gets no query gradient; keys of the sequence
    # without query rows get none either
    assert (dq[5] == 0).all() and (dk[3:5] == 0).all() and (dv[3:5] == 0).all()


def test_varlen_gradients_equal_the_batched_ones_for_equal_lengths():
    B, N, Hq, Hkv, d = 3, 5, 4, 2, 3
    q, k, v, cu_q, cu_k = make_varlen([N] * B, [N] * B, Hq, Hkv, d, seed=102)
    do = make_varlen([N] * B, [N] * B, Hq, Hkv, d, seed=103)[0]
    for causal in (False, True):
        a = oracle.attention_backward_varlen(q, k, v, do, cu_q, cu_k, 0.3, causal)
        b = oracle.attention_backward(q.reshape(B, N, Hq, d), k.reshape(B, N, Hkv, d),
                                      v.reshape(B, N, Hkv, d), do.reshape(B, N, Hq, d), 0.3, causal)
        np.testing.assert_allclose(a[0], b[0].reshape(B * N, Hq, d), rtol=0, atol=1e-14)
        np.testing.assert_allclose(a[1], b[1].reshape(B * N, Hkv, d), rtol=0, atol=1e-14)
        np.testing.assert_allclose(a[2], b[2].reshape(B * N, Hkv, d), rtol=0, atol=1e-14)
        np.testing.assert_allclose(a[3], b[3].transpose(1, 0, 2).reshape(Hq, B * N), rtol=0, atol=1e-14)
