"""Pins for the oracle's score variants: sliding window, ALiBi, softcap.

The hysenlabs.com page lists ``window_size`` and ``alibi_slopes`` among the
interface parameters and dates sliding windows (2.3), ALiBi (2.4) and
softcapping (2.6) in its version history ("Von 2.0 bis 2.7").  Each variant
is pinned against the pure-Python brute force, PyTorch's fp64 SDPA with an
additive float mask, and special cases that reduce to known results.
"""

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import oracle.exact as oa
from attn_workloads import make_qkv
from tests._bruteforce import brute_attention

SHAPES = [  # (B, Hq, Hkv, Nq, Nk, d, causal)
    (1, 2, 1, 6, 9, 4, True),
    (1, 2, 2, 7, 7, 3, False),
    (2, 4, 2, 5, 8, 4, False),
    (1, 3, 1, 8, 5, 2, True),
]
VARIANTS = [  # (left, right, slopes?, cap)
    (2, -1, False, 0.0),
    (-1, 1, False, 0.0),
    (1, 2, False, 0.0),
    (0, 0, False, 0.0),
    (-1, -1, True, 0.0),
    (3, 0, True, 0.0),
    (-1, -1, False, 1.5),
    (2, 1, True, 0.8),
]


def _f64(t):
    return t.to(torch.float64).numpy()


def _slopes(Hq):
    return np.float32(2.0) ** -np.arange(1, Hq + 1, dtype=np.float32)


@pytest.mark.parametrize("shape", SHAPES, ids=str)
@pytest.mark.parametrize("var", VARIANTS, ids=str)
def test_variants_match_brute_force(shape, var):
    B, Hq, Hkv, Nq, Nk, d, causal = shape
    left, right, use_slopes, cap = var
    q, k, v = make_qkv(B, Nq, Nk, Hq, Hkv, d, "bf16", 1.0, 40 + SHAPES.index(shape))
    slopes = _slopes(Hq) if use_slopes else None
    sc = 0.6
    O, lse = oracle.attention(q, k, v, sc, causal, window=(left, right), alibi_slopes=slopes,
                              softcap=cap)
    Ob, lb = brute_attention(_f64(q).tolist(), _f64(k).tolist(), _f64(v).tolist(),
                             float(np.float32(sc)), causal, left, right,
                             None if slopes is None else [float(x) for x in slopes],
                             float(np.float32(cap)))
    Ob, lb = np.array(Ob), np.array(lb)
    assert np.abs(O - Ob).max() <= 1e-13
    fin = np.isfinite(lb)
    assert np.array_equal(fin, np.isfinite(lse)) and np.all(lse[~fin] == -np.inf)
    assert np.abs(lse[fin] - lb[fin]).max(initial=0.0) <= 1e-13


@pytest.mark.parametrize("var", [(2, -1), (-1, 2), (3, 1), (0, 4)], ids=str)
@pytest.mark.parametrize("use_slopes", [False, True])
def test_window_and_alibi_match_sdpa_with_float_mask(var, use_slopes):
    B, Hq, Hkv, N, d = 2, 4, 2, 12, 8
    q, k, v = make_qkv(B, N, N, Hq, Hkv, d, "bf16", 1.0, 50)
    slopes = _slopes(Hq) if use_slopes else np.zeros(Hq, dtype=np.float32)
    left, right = var
    sc = 0.4
    O, lse = oracle.attention(q, k, v, sc, False, window=var,
                              alibi_slopes=slopes if use_slopes else None)
    i = torch.arange(N, dtype=torch.float64)[:, None]
    j = torch.arange(N, dtype=torch.float64)[None, :]
    vis = torch.ones(N, N, dtype=torch.bool)
    if left >= 0:
        vis &= j >= i - left
    if right >= 0:
        vis &= j <= i + right
    bias = -torch.tensor(slopes, dtype=torch.float64)[:, None, None] * (i - j).abs()
    mask = bias.masked_fill(~vis, float("-inf"))[None]  # [1, Hq, N, N]
    t = [x.to(torch.float64).transpose(1, 2) for x in (q, k, v)]
    ref = F.scaled_dot_product_attention(t[0], t[1], t[2], attn_mask=mask,
                                         scale=float(np.float32(sc)), enable_gqa=True)
    assert np.abs(O - ref.transpose(1, 2).numpy()).max() <= 1e-12


def test_window_zero_width_is_the_diagonal_key():
    q, k, v = make_qkv(1, 6, 10, 2, 1, 4, "bf16", 1.0, 51)
    O, lse = oracle.attention(q, k, v, 0.5, False, window=(0, 0))
    vv = _f64(v)
    for i in range(6):
        assert np.array_equal(O[0, i, 0], vv[0, i + 4, 0])


def test_wide_window_zero_slope_and_huge_cap_change_nothing():
    q, k, v = make_qkv(1, 9, 9, 2, 2, 8, "bf16", 1.0, 52)
    O0, l0 = oracle.attention(q, k, v, 0.3, True)
    O1, l1 = oracle.attention(q, k, v, 0.3, True, window=(9, 9), alibi_slopes=np.zeros(2))
    assert np.array_equal(O0, O1) and np.array_equal(l0, l1)
    O2, l2 = oracle.attention(q, k, v, 0.3, True, softcap=1e6)
    assert np.abs(O2 - O0).max() <= 1e-9 and np.abs(l2 - l0).max() <= 1e-9


def test_softcap_closed_form():
    # one query, two keys, d = 1: weights softmax(cap * tanh(s_j / cap))
    q = np.array([[[[1.5]]]])
    k = np.array([[[[2.0]], [[-1.0]]]])
    v = np.array([[[[1.0]], [[0.0]]]])
    cap = 1.25
    O, lse = oracle.attention(q, k, v, 1.0, False, softcap=cap)
    t = cap * np.tanh(np.array([3.0, -1.5]) / cap)
    assert abs(O[0, 0, 0, 0] - math.exp(t[0]) / np.exp(t).sum()) <= 1e-15
    assert abs(lse[0, 0, 0] - math.log(np.exp(t).sum())) <= 1e-14


def test_steep_alibi_picks_the_diagonal_key():
    q, k, v = make_qkv(1, 5, 7, 1, 1, 4, "bf16", 1.0, 53)
    O, _ = oracle.attention(q, k, v, 0.1, False, alibi_slopes=np.array([60.0], dtype=np.float32))
    vv = _f64(v)
    for i in range(5):
        assert np.abs(O[0, i, 0] - vv[0, i + 2, 0]).max() <= 1e-20 + 8 * math.exp(-55.0)


def test_alibi_zero_q_closed_form():
    # zero queries: weights proportional to exp(-slope * |i + diag - j|)
    _, k, v = make_qkv(1, 4, 6, 1, 1, 2, "bf16", 1.0, 54)
    q = torch.zeros(1, 4, 1, 2, dtype=torch.bfloat16)
    sl = 0.75
    O, _ = oracle.attention(q, k, v, 1.0, False, alibi_slopes=np.array([sl], dtype=np.float32))
    vv = _f64(v)[0, :, 0]
    for i in range(4):
        w = np.exp(-sl * np.abs(i + 2 - np.arange(6)))
        assert np.abs(O[0, i, 0] - (w[:, None] * vv).sum(0) / w.sum()).max() <= 1e-14


def test_planted_variant_mistakes_are_caught(monkeypatch):
    # An off-by-one window and a signed (not absolute) ALiBi distance.
    real = oa.visible_range

    def shifted(i, Nq, Nk, causal, window=(-1, -1)):
        lo, hi = real(i, Nq, Nk, causal, window)
        return min(lo + 1, hi), hi

    q, k, v = make_qkv(1, 6, 9, 2, 1, 4, "bf16", 1.0, 55)
    brute = brute_attention(_f64(q).tolist(), _f64(k).tolist(), _f64(v).tolist(),
                            float(np.float32(0.6)), False, 2, 1)
    monkeypatch.setattr(oa, "visible_range", shifted)
    O, _ = oracle.attention(q, k, v, 0.6, False, window=(2, 1))
    monkeypatch.undo()
    assert np.abs(O - np.array(brute[0])).max() > 1e-3

    real_rows = oa._rows_of_one_head

    def signed(qh, kg, vg, sigma, rows, Nq, Nk, causal, want_p, window=(-1, -1), slope=0.0,
               softcap=0.0):
        O, lse, S, P = real_rows(qh, kg, vg, sigma, rows, Nq, Nk, causal, want_p, window, 0.0, softcap)
        # recompute with a signed distance
        Sg = sigma * (qh[rows] @ kg.T) - slope * (np.asarray(rows)[:, None] + Nk - Nq - np.arange(Nk))
        Pg = np.exp(Sg - Sg.max(1, keepdims=True))
        Pg /= Pg.sum(1, keepdims=True)
        return Pg @ vg, lse, S, P

    monkeypatch.setattr(oa, "_rows_of_one_head", signed)
    sl = np.array([0.5, 0.25], dtype=np.float32)
    O2, _ = oracle.attention(q, k, v, 0.6, False, alibi_slopes=sl)
    monkeypatch.undo()
    brute2 = brute_attention(_f64(q).tolist(), _f64(k).tolist(), _f64(v).tolist(),
                             float(np.float32(0.6)), False, slopes=[0.5, 0.25])
    assert np.abs(O2 - np.array(brute2[0])).max() > 1e-3
