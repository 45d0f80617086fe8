"""Pins of the oracle's block-sparse attention (CPU only).

The block mask keeps or drops whole (query block, key block) pairs of the
score matrix (block sparsity, named among the features of FlexAttention's
new backend in the liora.io item).  Checked against: the pure-Python brute
force with the mask written out as an element predicate of its own (block
sizes 1 to 4 on tiny shapes, causal with Nq != Nk both ways, GQA, head-shared
and per-head masks, rows that keep no key); fp64 scaled_dot_product_attention
with the expanded boolean mask; documents on the block diagonal against the
packed variable-length oracle; and the dense oracle for an all-ones mask.
Planted mistakes (transposed flags, flags shifted by one key block, every
head reading head 0's flags) must fail the brute-force pin."""

import math

import numpy as np
import pytest
import torch

import oracle
from attn_workloads import make_block_mask, make_qkv, make_varlen
from _bruteforce import brute_attention

# (B, Nq, Nk, Hq, Hkv, d, block, Hm, causal)
CASES = [
    (1, 5, 7, 2, 1, 4, 2, 1, False),
    (1, 5, 7, 2, 1, 4, 2, 2, True),   # Nq < Nk: bottom-right causal
    (2, 7, 4, 4, 2, 3, 3, 4, True),   # Nq > Nk: rows above the first key
    (1, 6, 6, 2, 2, 5, 4, 1, False),  # ragged last block
    (1, 4, 5, 1, 1, 3, 1, 1, False),  # block 1: an element mask
    (2, 8, 8, 4, 1, 2, 2, 4, True),   # MQA
]


def lists(x):
    return x.double().tolist()


def brute_block_sparse(q, k, v, mask, scale, causal, block):
    m = (np.asarray(mask) != 0).tolist()
    shared = len(m[0]) == 1

    def keep(b, h, i, j):
        return m[b][0 if shared else h][i // block][j // block]

    O, L = brute_attention(lists(q), lists(k), lists(v), scale, causal, keep=keep)
    return np.array(O), np.array(L)


def draw(case, seed):
    B, Nq, Nk, Hq, Hkv, d, block, Hm, causal = case
    q, k, v = make_qkv(B, Nq, Nk, Hq, Hkv, d, "bf16", 1.0, seed)
    mask = make_block_mask(B, Hm, -(-Nq // block), -(-Nk // block), 0.5, seed + 1)
    mask[0, 0, 0, :] = 0  # the first query block of (0, 0) keeps no key
    return q, k, v, mask


@pytest.mark.parametrize("case", CASES)
def test_matches_bruteforce(case):
    B, Nq, Nk, Hq, Hkv, d, block, Hm, causal = case
    q, k, v, mask = draw(case, 21)
    scale = float(np.float32(1 / math.sqrt(d)))
    O, L = oracle.attention_block_sparse(q, k, v, mask, scale, causal, block=block)
    Ob, Lb = brute_block_sparse(q, k, v, mask, scale, causal, block)
    np.testing.assert_allclose(O, Ob, rtol=0, atol=1e-12)
    fin = np.isfinite(Lb)
    assert (np.isfinite(L) == fin).all()
    np.testing.assert_allclose(L[fin], Lb[fin], rtol=0, atol=1e-12)
    # the query block with no kept key: zero output, -inf logsumexp
    assert (O[0, :block, 0, :] == 0).all() and np.isneginf(L[0, 0, :block]).all()


@pytest.mark.parametrize("causal", [False, True])
def test_matches_sdpa_with_the_expanded_mask(causal):
    B, Nq, Nk, Hq, Hkv, d, block = 2, 9, 9, 4, 2, 8, 2
    q, k, v = make_qkv(B, Nq, Nk, Hq, Hkv, d, "fp16", 1.0, 31)
    mask = make_block_mask(B, Hq, 5, 5, 0.6, 32)
    mask[1, 2, 1, :] = 0  # rows 2-3 of (1, head 2) keep no key
    scale = float(np.float32(0.3))
    O, L = oracle.attention_block_sparse(q, k, v, mask, scale, causal, block=block)
    # torch's own path: [B, H, N, d] fp64, KV heads repeated per group, the
    # boolean mask expanded with repeat_interleave, causal as a lower triangle
    em = mask.bool().repeat_interleave(block, 2)[:, :, :Nq].repeat_interleave(block, 3)[..., :Nk]
    if causal:
        em = em & torch.ones(Nq, Nk, dtype=torch.bool).tril(Nk - Nq)
    qt = q.double().permute(0, 2, 1, 3)
    kt = k.double().permute(0, 2, 1, 3).repeat_interleave(Hq // Hkv, 1)
    vt = v.double().permute(0, 2, 1, 3).repeat_interleave(Hq // Hkv, 1)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=em, scale=scale)
    ref = ref.permute(0, 2, 1, 3).numpy()
    has = em.any(-1).permute(0, 2, 1).numpy()  # [B, Nq, Hq]: rows that keep a key
    assert has.any() and (~has).any()
    np.testing.assert_allclose(O[has], ref[has], rtol=0, atol=1e-12)
    assert (O[~has] == 0).all()
    s = torch.where(em, scale * (qt @ kt.transpose(-1, -2)), torch.tensor(-math.inf, dtype=torch.float64))
    np.testing.assert_allclose(L, torch.logsumexp(s, -1).numpy(), rtol=0, atol=1e-12)


def test_all_ones_equals_the_dense_oracle():
    q, k, v = make_qkv(2, 7, 9, 4, 2, 6, "bf16", 1.0, 41)
    for causal in (False, True):
        O, L = oracle.attention_block_sparse(q, k, v, np.ones((2, 1, 4, 5)), 0.4, causal, block=2)
        Od, Ld = oracle.attention(q, k, v, 0.4, causal)
        np.testing.assert_array_equal(O, Od)
        np.testing.assert_array_equal(L, Ld)


@pytest.mark.parametrize("causal", [False, True])
def test_block_diagonal_documents_equal_varlen(causal):
    # documents of 2, 4 and 2 blocks of 2 rows packed into one sequence
    block, docs, Hq, Hkv, d = 2, [4, 8, 4], 2, 1, 4
    q, k, v, cu_q, cu_k = make_varlen(docs, docs, Hq, Hkv, d, "bf16", 1.0, seed=51)
    N = sum(docs)
    nb = N // block
    mask = np.zeros((1, 1, nb, nb), dtype=np.uint8)
    for s0, s1 in zip(cu_q[:-1].tolist(), cu_q[1:].tolist()):
        mask[0, 0, s0 // block:s1 // block, s0 // block:s1 // block] = 1
    O, L = oracle.attention_block_sparse(q[None], k[None], v[None], mask, 0.5, causal, block=block)
    Ov, Lv = oracle.attention_varlen(q, k, v, cu_q, cu_k, 0.5, causal)
    np.testing.assert_allclose(O[0], Ov, rtol=0, atol=1e-13)
    np.testing.assert_allclose(L[0], Lv, rtol=0, atol=1e-13)


@pytest.mark.parametrize("mistake", ["transposed", "shifted_key_block", "head0_for_all"])
def test_planted_mask_mistakes_fail_the_pin(mistake):
    case = (1, 8, 8, 2, 1, 4, 2, 2, False)
    B, Nq, Nk, Hq, Hkv, d, block, Hm, causal = case
    q, k, v, mask = draw(case, 61)
    mask[0, 1] = 1 - mask[0, 0]  # heads with different flags
    m = mask.numpy()
    if mistake == "transposed":
        wrong = m.transpose(0, 1, 3, 2)
    elif mistake == "shifted_key_block":
        wrong = np.roll(m, 1, axis=3)
    else:
        wrong = np.repeat(m[:, :1], Hm, axis=1)
    assert (wrong != m).any()
    Ow, _ = oracle.attention_block_sparse(q, k, v, wrong, 0.5, causal, block=block)
    Ob, _ = brute_block_sparse(q, k, v, mask, 0.5, causal, block)
    assert np.abs(Ow - Ob).max() > 1e-3


def test_rejects_a_mask_of_the_wrong_shape():
    q, k, v = make_qkv(1, 5, 5, 2, 1, 4, "bf16", 1.0, 71)
    with pytest.raises(ValueError):
        oracle.attention_block_sparse(q, k, v, np.ones((1, 3, 3, 3)), 0.5, False, block=2)
    with pytest.raises(ValueError):
        oracle.attention_block_sparse(q, k, v, np.ones((1, 1, 2, 3)), 0.5, False, block=2)


@pytest.mark.parametrize("causal", [False, True])
def test_selected_rows_equal_the_full_evaluation(causal):
    case = (2, 11, 9, 4, 2, 3, 3, 4, causal)
    q, k, v, mask = draw(case, 81)
    O, L = oracle.attention_block_sparse(q, k, v, mask, 0.7, causal, block=3)
    for b, h, rows in ((0, 0, [0, 1, 2]), (1, 3, [10, 4, 7]), (1, 1, range(11))):
        Or, Lr = oracle.attention_block_sparse_rows(q, k, v, mask, 0.7, causal, b, h, rows, block=3)
        np.testing.assert_array_equal(Or, O[b, list(rows), h, :])
        np.testing.assert_array_equal(Lr, L[b, h, list(rows)])


# ---------------------------------------------------------------------------
# Gradients of the block-sparse attention (attention_backward with a mask)
# ---------------------------------------------------------------------------
BWD_CASES = [  # (B, Nq, Nk, Hq, Hkv, d, block, Hm, causal)
    (1, 5, 7, 2, 1, 3, 2, 2, False),
    (1, 6, 4, 2, 2, 2, 2, 1, True),   # Nq > Nk: rows above the first key
    (2, 4, 6, 2, 1, 2, 3, 2, True),
]


def bs_loss(q, k, v, do, mask, scale, causal, block):
    O, _ = oracle.attention_block_sparse(q, k, v, mask, scale, causal, block=block)
    return float((O * do).sum())


def bs_finite_difference(q, k, v, do, mask, scale, causal, block, eps=1e-6):
    grads = []
    for which in range(3):
        args = [q.copy(), k.copy(), v.copy()]
        x = args[which]
        g = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            x0 = x[idx]
            x[idx] = x0 + eps
            lp = bs_loss(*args, do, mask, scale, causal, block)
            x[idx] = x0 - eps
            lm = bs_loss(*args, do, mask, scale, causal, block)
            x[idx] = x0
            g[idx] = (lp - lm) / (2 * eps)
        grads.append(g)
    return grads


def bwd_case(case, seed):
    B, Nq, Nk, Hq, Hkv, d, block, Hm, causal = case
    rng = np.random.default_rng(seed)
    q, k, v = (rng.standard_normal(s) for s in ((B, Nq, Hq, d), (B, Nk, Hkv, d), (B, Nk, Hkv, d)))
    do = rng.standard_normal((B, Nq, Hq, d))
    mask = (rng.random((B, Hm, -(-Nq // block), -(-Nk // block))) < 0.6).astype(np.uint8)
    mask[0, 0, 0, :] = 0  # a query block that keeps no key
    return q, k, v, do, mask


@pytest.mark.parametrize("case", BWD_CASES, ids=str)
def test_block_sparse_gradients_match_finite_differences(case):
    q, k, v, do, mask = bwd_case(case, 91)
    causal, block = case[-1], case[6]
    dq, dk, dv, _ = oracle.attention_backward(q, k, v, do, 0.6, causal, block_mask=mask, block=block)
    fq, fk, fv = bs_finite_difference(q, k, v, do, mask, float(np.float32(0.6)), causal, block)
    for got, want in ((dq, fq), (dk, fk), (dv, fv)):
        assert np.abs(got - want).max() <= 1e-7
    assert (dq[0, :block, 0] == 0).all()  # rows that keep no key get no gradient


def test_block_sparse_gradients_match_sdpa_autograd():
    B, Nq, Nk, Hq, Hkv, d, block = 2, 9, 9, 4, 2, 5, 2
    rng = np.random.default_rng(92)
    q, k, v, do = (rng.standard_normal(s) for s in
                   ((B, Nq, Hq, d), (B, Nk, Hkv, d), (B, Nk, Hkv, d), (B, Nq, Hq, d)))
    mask = (rng.random((B, Hq, 5, 5)) < 0.5).astype(np.uint8)
    mask[..., 0] = 1  # every row keeps a key (SDPA gives NaN for rows that keep none)
    for causal in (False, True):
        dq, dk, dv, _ = oracle.attention_backward(q, k, v, do, 0.4, causal, block_mask=mask, block=block)
        em = torch.tensor(mask).bool().repeat_interleave(block, 2)[:, :, :Nq].repeat_interleave(block, 3)[..., :Nk]
        if causal:
            em = em & torch.ones(Nq, Nk, dtype=torch.bool).tril(Nk - Nq)
        t = [torch.tensor(x).transpose(1, 2).contiguous().requires_grad_(True) for x in (q, k, v)]
        kt = t[1].repeat_interleave(Hq // Hkv, 1)
        vt = t[2].repeat_interleave(Hq // Hkv, 1)
        out = torch.nn.functional.scaled_dot_product_attention(t[0], kt, vt, attn_mask=em,
                                                               scale=float(np.float32(0.4)))
        out.backward(torch.tensor(do).transpose(1, 2))
        for got, ref in zip((dq, dk, dv), t):
            np.testing.assert_allclose(got, ref.grad.transpose(1, 2).numpy(), rtol=0, atol=1e-12)


def test_all_ones_mask_gives_the_dense_gradients():
    rng = np.random.default_rng(93)
    q, k, v, do = (rng.standard_normal(s) for s in ((1, 5, 2, 3), (1, 6, 1, 3), (1, 6, 1, 3), (1, 5, 2, 3)))
    for causal in (False, True):
        a = oracle.attention_backward(q, k, v, do, 0.5, causal, block_mask=np.ones((1, 1, 3, 3)), block=2)
        b = oracle.attention_backward(q, k, v, do, 0.5, causal)
        for x, y in zip(a, b):
            np.testing.assert_array_equal(x, y)


def test_planted_mask_mistake_fails_the_gradient_pin():
    case = BWD_CASES[0]
    q, k, v, do, mask = bwd_case(case, 94)
    mask[0, 1] = 1 - mask[0, 0]
    wrong = np.roll(mask, 1, axis=3)
    dq, dk, dv, _ = oracle.attention_backward(q, k, v, do, 0.6, False, block_mask=wrong, block=2)
    fq, fk, fv = bs_finite_difference(q, k, v, do, mask, float(np.float32(0.6)), False, 2)
    assert max(np.abs(dq - fq).max(), np.abs(dk - fk).max(), np.abs(dv - fv).max()) > 1e-3
