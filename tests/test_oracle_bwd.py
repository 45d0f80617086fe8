"""Pins of the fp64 backward oracle (CPU only).

The gradients are the derivatives of the forward definition, so they are
pinned against things that do not share the oracle's chain-rule code:
central finite differences of the (separately pinned) forward oracle,
PyTorch's own autograd through its fp64 scaled-dot-product attention on the
CPU (the library routine the tokenwerk.de page uses in its example), and
identities of the softmax Jacobian.  Planted mistakes show that each kind of
error is caught.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import oracle.exact as oe

TINY = [  # (B, Hq, Hkv, Nq, Nk, d, causal)
    (1, 1, 1, 1, 1, 2, False),
    (1, 2, 1, 5, 7, 4, True),    # Nq < Nk, GQA
    (1, 2, 2, 6, 3, 3, True),    # Nq > Nk: rows with no visible key
    (2, 4, 2, 4, 4, 4, False),
    (1, 3, 1, 5, 5, 2, True),    # MQA
]


def rand_case(case, seed):
    B, Hq, Hkv, Nq, Nk, d, causal = case
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Nq, Hq, d))
    k = rng.standard_normal((B, Nk, Hkv, d))
    v = rng.standard_normal((B, Nk, Hkv, d))
    do = rng.standard_normal((B, Nq, Hq, d))
    return q, k, v, do


def loss(q, k, v, do, scale, causal):
    O, _ = oracle.attention(q, k, v, scale, causal)
    return float((O * do).sum())


def finite_difference(q, k, v, do, scale, causal, eps=1e-6):
    grads = []
    for which in range(3):
        args = [q.copy(), k.copy(), v.copy()]
        x = args[which]
        g = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            x0 = x[idx]
            x[idx] = x0 + eps
            lp = loss(*args, do, scale, causal)
            x[idx] = x0 - eps
            lm = loss(*args, do, scale, causal)
            x[idx] = x0
            g[idx] = (lp - lm) / (2 * eps)
        grads.append(g)
    return grads


@pytest.mark.parametrize("case", TINY, ids=str)
@pytest.mark.parametrize("scale", [0.7, -0.4])
def test_backward_matches_finite_differences(case, scale):
    q, k, v, do = rand_case(case, 7)
    dq, dk, dv, _ = oracle.attention_backward(q, k, v, do, scale, case[-1])
    fq, fk, fv = finite_difference(q, k, v, do, float(np.float32(scale)), case[-1])
    for got, want in ((dq, fq), (dk, fk), (dv, fv)):
        assert np.abs(got - want).max() <= 1e-7


def sdpa_grads(q, k, v, do, scale, causal):
    B, Nq, Hq, d = q.shape
    Hkv = k.shape[2]
    t = [torch.tensor(x).transpose(1, 2).contiguous().requires_grad_(True) for x in (q, k, v)]
    out = torch.nn.functional.scaled_dot_product_attention(
        t[0], t[1], t[2], is_causal=causal, scale=float(np.float32(scale)), enable_gqa=Hkv != Hq)
    out.backward(torch.tensor(do).transpose(1, 2))
    return [x.grad.transpose(1, 2).numpy() for x in t]


@pytest.mark.parametrize("case", [(1, 2, 2, 9, 9, 8, True), (2, 4, 1, 12, 12, 16, False),
                                  (1, 8, 2, 33, 33, 8, True)], ids=str)
def test_backward_matches_torch_autograd_fp64(case):
    # Nq == Nk only: SDPA's is_causal is the top-left mask, which equals the
    # bottom-right one exactly when the lengths agree.
    q, k, v, do = rand_case(case, 11)
    scale = 1.0 / math.sqrt(case[5])
    dq, dk, dv, _ = oracle.attention_backward(q, k, v, do, scale, case[-1])
    tq, tk, tv = sdpa_grads(q, k, v, do, scale, case[-1])
    for got, want in ((dq, tq), (dk, tk), (dv, tv)):
        assert np.abs(got - want).max() <= 1e-12


@pytest.mark.parametrize("case", TINY[1:], ids=str)
def test_backward_identities(case):
    B, Hq, Hkv, Nq, Nk, d, causal = case
    q, k, v, do = rand_case(case, 3)
    scale = 0.6
    dq, dk, dv, D = oracle.attention_backward(q, k, v, do, scale, causal)
    O, _ = oracle.attention(q, k, v, scale, causal)
    G = Hq // Hkv
    # D is the row-wise dot product of dout and out.
    assert np.abs(D - np.einsum("bihc,bihc->bhi", do, O)).max() <= 1e-12
    # Every row of dS sums to zero, so the key gradients of a head sum to 0.
    assert np.abs(dk.sum(axis=1)).max() <= 1e-12
    # Rows of P sum to 1 (0 for rows with no visible key): the value
    # gradients of a KV head sum to the dout rows of its query heads.
    seen = np.array([oracle.allowed_keys(i, Nq, Nk, causal) > 0 for i in range(Nq)])
    want = (do * seen[None, :, None, None]).reshape(B, Nq, Hkv, G, d).sum(axis=(1, 3))
    assert np.abs(dv.sum(axis=1) - want).max() <= 1e-12
    # Constant V: the output does not depend on q or k.
    vc = np.ones_like(v) * 0.3
    dq0, dk0, _, _ = oracle.attention_backward(q, k, vc, do, scale, causal)
    assert np.abs(dq0).max() <= 1e-12 and np.abs(dk0).max() <= 1e-12
    # Zero upstream gradient: zero gradients.
    z = oracle.attention_backward(q, k, v, np.zeros_like(do), scale, causal)
    assert all(np.abs(x).max() == 0.0 for x in z)


def test_backward_accepts_torch_low_precision_inputs():
    case = (1, 2, 1, 5, 7, 4, True)
    q, k, v, do = (torch.tensor(x).to(torch.bfloat16) for x in rand_case(case, 5))
    got = oracle.attention_backward(q, k, v, do, 0.5, True)
    want = oracle.attention_backward(*(x.double().numpy() for x in (q, k, v, do)), 0.5, True)
    for a, b in zip(got, want):
        assert np.array_equal(a, b)


# Planted mistakes: each must make at least one pin above fail.
def _no_delta(P, dP):
    return P * dP, (P * dP).sum(axis=1)


def _delta_sign(P, dP):
    D = (P * dP).sum(axis=1)
    return P * (dP + D[:, None]), D


def _transposed_jacobian(P, dP):
    D = (P * dP).sum(axis=0)
    return P * (dP - D[None, :]), (P * dP).sum(axis=1)


@pytest.mark.parametrize("mutant", [_no_delta, _delta_sign, _transposed_jacobian])
def test_planted_jacobian_mistakes_are_caught(monkeypatch, mutant):
    monkeypatch.setattr(oe, "_softmax_rows_backward", mutant)
    case = (1, 2, 1, 4, 4, 3, False)
    q, k, v, do = rand_case(case, 9)
    dq, dk, dv, _ = oracle.attention_backward(q, k, v, do, 0.7, False)
    monkeypatch.undo()
    fq, fk, fv = finite_difference(q, k, v, do, float(np.float32(0.7)), False)
    assert max(np.abs(dq - fq).max(), np.abs(dk - fk).max()) > 1e-4


def test_planted_grouping_mistake_is_caught(monkeypatch):
    # GQA: a wrong query-head -> KV-head map breaks the agreement with autograd.
    monkeypatch.setattr(oe, "kv_head_of", lambda h, Hq, Hkv: h % Hkv)
    case = (1, 4, 2, 6, 6, 4, False)
    q, k, v, do = rand_case(case, 13)
    dq, dk, dv, _ = oracle.attention_backward(q, k, v, do, 0.5, False)
    monkeypatch.undo()
    tq, tk, tv = sdpa_grads(q, k, v, do, 0.5, False)
    assert np.abs(dk - tk).max() > 1e-3


def test_planted_mask_mistake_is_caught(monkeypatch):
    # Causal mask aligned top-left instead of bottom-right (Nq < Nk).
    monkeypatch.setattr(oe, "allowed_keys",
                        lambda i, Nq, Nk, causal: Nk if not causal else int(max(0, min(Nk, i + 1))))
    case = (1, 1, 1, 3, 6, 2, True)
    q, k, v, do = rand_case(case, 17)
    dq, dk, dv, _ = oracle.attention_backward(q, k, v, do, 0.8, True)
    monkeypatch.undo()
    fq, fk, fv = finite_difference(q, k, v, do, float(np.float32(0.8)), True)
    assert np.abs(dv - fv).max() > 1e-3


# ---------------------------------------------------------------------------
# Score variants (window, ALiBi, softcap) in the gradients
# ---------------------------------------------------------------------------
VAR_CASES = [  # (B, Hq, Hkv, Nq, Nk, d, causal, window, alibi, cap)
    (1, 2, 1, 5, 7, 3, True, (2, 0), False, 0.0),
    (1, 2, 2, 6, 4, 2, False, (1, 2), True, 0.0),
    (1, 2, 1, 4, 6, 3, False, (-1, -1), False, 1.5),
    (1, 2, 2, 5, 5, 2, True, (3, -1), True, 2.0),
]


def variant_loss(q, k, v, do, scale, causal, window, slopes, cap):
    O, _ = oracle.attention(q, k, v, scale, causal, window=window, alibi_slopes=slopes, softcap=cap)
    return float((O * do).sum())


@pytest.mark.parametrize("case", VAR_CASES, ids=str)
def test_variant_gradients_match_finite_differences(case):
    B, Hq, Hkv, Nq, Nk, d, causal, window, alibi, cap = case
    q, k, v, do = rand_case((B, Hq, Hkv, Nq, Nk, d, causal), 11)
    slopes = np.array([0.5, 0.25][:Hq], dtype=np.float32) if alibi else None
    dq, dk, dv, _ = oracle.attention_backward(q, k, v, do, 0.7, causal, window=window,
                                              alibi_slopes=slopes, softcap=cap)
    eps = 1e-6
    sc = float(np.float32(0.7))
    for x, g in ((q, dq), (k, dk), (v, dv)):
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            x0 = x[idx]
            x[idx] = x0 + eps
            lp = variant_loss(q, k, v, do, sc, causal, window, slopes, cap)
            x[idx] = x0 - eps
            lm = variant_loss(q, k, v, do, sc, causal, window, slopes, cap)
            x[idx] = x0
            fd[idx] = (lp - lm) / (2 * eps)
        assert np.abs(g - fd).max() <= 1e-7


def test_window_and_alibi_gradients_match_sdpa_autograd():
    B, Hq, Hkv, Nq, Nk, d = 2, 4, 2, 7, 9, 3
    rng = np.random.default_rng(12)
    q, k, v, do = (rng.standard_normal(s) for s in
                   ((B, Nq, Hq, d), (B, Nk, Hkv, d), (B, Nk, Hkv, d), (B, Nq, Hq, d)))
    slopes = np.array([0.5, 0.25, 0.125, 0.0625], dtype=np.float32)
    left, right = 3, 1
    dq, dk, dv, _ = oracle.attention_backward(q, k, v, do, 0.6, False, window=(left, right),
                                              alibi_slopes=slopes)
    i = torch.arange(Nq)[:, None] + (Nk - Nq)
    j = torch.arange(Nk)[None, :]
    keep = (j >= i - left) & (j <= i + right)
    bias = -torch.tensor(slopes, dtype=torch.float64)[:, None, None] * (i - j).abs()
    bias = torch.where(keep, bias, torch.tensor(-math.inf, dtype=torch.float64))
    t = [torch.tensor(x).transpose(1, 2).contiguous().requires_grad_(True) for x in (q, k, v)]
    kt = t[1].repeat_interleave(Hq // Hkv, 1)
    vt = t[2].repeat_interleave(Hq // Hkv, 1)
    out = torch.nn.functional.scaled_dot_product_attention(t[0], kt, vt, attn_mask=bias[None],
                                                           scale=float(np.float32(0.6)))
    out.backward(torch.tensor(do).transpose(1, 2))
    for got, ref in zip((dq, dk, dv), t):
        np.testing.assert_allclose(got, ref.grad.transpose(1, 2).numpy(), rtol=0, atol=1e-12)


def test_softcap_gradient_without_its_derivative_fails_the_pin():
    case = VAR_CASES[2]
    B, Hq, Hkv, Nq, Nk, d, causal, window, alibi, cap = case
    q, k, v, do = rand_case((B, Hq, Hkv, Nq, Nk, d, causal), 13)
    good = oracle.attention_backward(q, k, v, do, 0.7, causal, softcap=cap)
    # planted: the softcap's probabilities, but dS not multiplied by 1 - tanh^2
    P = oracle.attention(q, k, v, 0.7, causal, softcap=cap, return_probs=True)[2]
    sigma = float(np.float32(0.7))
    dq_wrong = np.zeros_like(q)
    for h in range(Hq):
        g = h * Hkv // Hq
        dP = do[0, :, h, :] @ v[0, :, g, :].T
        D = (P[0, h] * dP).sum(1, keepdims=True)
        dq_wrong[0, :, h, :] = sigma * ((P[0, h] * (dP - D)) @ k[0, :, g, :])
    assert np.abs(dq_wrong - good[0]).max() > 1e-3
