"""Pins for the fp64 oracle (CPU only).

Each test checks the oracle against something other than itself: a
pure-Python brute force, closed forms, invariants of softmax attention, the
pages' own size arithmetic, and PyTorch's CPU scaled-dot-product attention
(the function the tokenwerk.de page's example calls).  The mutation tests at
the end plant plausible mistakes in the oracle and check that the pins catch
them.
"""

import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import oracle.exact as oa
from attn_workloads import make_qkv
from tests._bruteforce import brute_attention

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

# (B, Hq, Hkv, Nq, Nk, d, causal)
TINY = [
    (1, 1, 1, 1, 1, 1, False),
    (1, 2, 1, 3, 5, 4, False),
    (2, 4, 2, 7, 7, 8, False),
    (1, 1, 1, 4, 9, 2, True),    # Nq < Nk: bottom-right alignment
    (1, 2, 2, 5, 3, 4, True),    # Nq > Nk: rows 0, 1 see no key
    (2, 6, 3, 6, 6, 3, True),    # GQA, causal, square
    (1, 4, 1, 5, 8, 5, False),   # MQA
]


def _inputs(shape, seed, dtype="bf16", sigma=1.0):
    B, Hq, Hkv, Nq, Nk, d, _ = shape
    return make_qkv(B, Nq, Nk, Hq, Hkv, d, dtype, sigma, seed)


def _f64(t):
    return t.to(torch.float64).numpy()


@pytest.mark.parametrize("shape", TINY)
@pytest.mark.parametrize("scale", [None, 0.0, -0.7, 2.25])
def test_oracle_matches_brute_force(shape, scale):
    q, k, v = _inputs(shape, seed=100 + TINY.index(shape))
    d = shape[5]
    sc = 1.0 / math.sqrt(d) if scale is None else scale
    sigma = float(np.float32(sc))
    O, lse = oracle.attention(q, k, v, sc, shape[6])
    Ob, lseb = brute_attention(_f64(q).tolist(), _f64(k).tolist(), _f64(v).tolist(), sigma, shape[6])
    Ob = np.array(Ob)
    lseb = np.array(lseb)
    assert np.max(np.abs(O - Ob)) <= 1e-13
    fin = np.isfinite(lseb)
    assert np.array_equal(fin, np.isfinite(lse))
    assert np.all(lse[~fin] == -np.inf)
    assert np.max(np.abs(lse[fin] - lseb[fin]), initial=0.0) <= 1e-13


@pytest.mark.parametrize("causal", [False, True])
def test_softmax_rows_sum_to_one(causal):
    q, k, v = make_qkv(2, 33, 40, 4, 2, 16, "bf16", 1.0, 7)
    _, _, P = oracle.attention(q, k, v, 0.25, causal, return_probs=True)
    sums = P.sum(axis=-1)
    assert np.max(np.abs(sums - 1.0)) <= 1e-14
    assert np.all(P >= 0)
    if causal:  # masked keys carry exactly zero weight
        Nq, Nk = 33, 40
        i = np.arange(Nq)[:, None]
        j = np.arange(Nk)[None, :]
        assert np.all(P[..., (j - i) > (Nk - Nq)] == 0.0)


@pytest.mark.parametrize("causal,Nq,Nk", [(False, 9, 9), (True, 9, 9), (True, 6, 11), (True, 11, 6)])
def test_zero_q_gives_mean_of_visible_v(causal, Nq, Nk):
    _, k, v = make_qkv(1, Nq, Nk, 2, 1, 8, "bf16", 1.0, 11)
    q = torch.zeros(1, Nq, 2, 8, dtype=torch.bfloat16)
    O, lse = oracle.attention(q, k, v, 0.5, causal)
    vv = _f64(v)[0, :, 0, :]
    for i in range(Nq):
        n = Nk if not causal else max(0, min(Nk, i + Nk - Nq + 1))
        for h in range(2):
            if n == 0:
                assert np.all(O[0, i, h] == 0.0) and lse[0, h, i] == -np.inf
            else:
                assert np.max(np.abs(O[0, i, h] - vv[:n].mean(axis=0))) <= 1e-13
                assert abs(lse[0, h, i] - math.log(n)) <= 1e-13


@pytest.mark.parametrize("d", [1, 8, 64])
def test_causal_row0_is_v0(d):
    q, k, v = make_qkv(2, 17, 17, 3, 3, d, "bf16", 1.0, 12)
    sc = 0.37
    O, lse = oracle.attention(q, k, v, sc, True)
    qq, kk, vv = _f64(q), _f64(k), _f64(v)
    sigma = float(np.float32(sc))
    for b in range(2):
        for h in range(3):
            assert np.array_equal(O[b, 0, h], vv[b, 0, h])
            assert abs(lse[b, h, 0] - sigma * float(qq[b, 0, h] @ kk[b, 0, h])) <= 1e-14


def test_one_hot_dominant_key():
    Nq, Nk, d = 5, 23, 16
    q, k, v = make_qkv(1, Nq, Nk, 1, 1, d, "bf16", 1.0, 13)
    qq = _f64(q)
    kk = _f64(k).copy()
    vv = _f64(v)
    scale = 1.0
    i, jstar = 3, 17
    # Other scores are |<q,k>| <~ 20 here; put key j* at a score gap >= 40.
    qi = qq[0, i, 0]
    others = np.abs(kk[0, :, 0] @ qi).max()
    c = (others + 60.0) / float(qi @ qi)
    kk[0, jstar, 0] = c * qi
    O, _ = oracle.attention(qq, kk, vv, scale, False)
    s = kk[0, :, 0] @ qi
    gap = s[jstar] - np.delete(s, jstar).max()
    assert gap >= 40.0
    assert np.max(np.abs(O[0, i, 0] - vv[0, jstar, 0])) <= Nk * math.exp(-40.0) * np.abs(vv).max() * 2


def test_pages_score_matrix_arithmetic():
    with open(os.path.join(GOLDEN, "score_matrix_sizes.json")) as f:
        g = json.load(f)
    for row in g["dense"]:
        N = row["N"]
        assert oracle.materialised_score_bytes(N, N, g["bytes_per_cell"]) == row["bytes"]
        assert row["bytes"] == row["cells"] * g["bytes_per_cell"]
        assert row["cells"] == N * N
    assert oracle.materialised_score_bytes(g["tile"]["rows"], g["tile"]["cols"], 2) == g["tile"]["bytes"]
    assert g["tile"]["bytes"] == 128 * 1024
    assert g["dense"][0]["bytes"] == 2 * 2**20 and g["dense"][1]["bytes"] == 32 * 2**20
    a, b = g["dense"]
    assert b["N"] == g["length_ratio"] * a["N"] and b["bytes"] == g["size_ratio"] * a["bytes"]
    # The oracle really writes out that matrix: one head at N = 1,024 has
    # 1,048,576 score cells.
    q, k, v = make_qkv(1, 1024, 1024, 1, 1, 4, "bf16", 1.0, 14)
    _, _, S = oracle.attention(q, k, v, 0.5, False, return_scores=True)
    assert S[0, 0].size == g["dense"][0]["cells"]
    assert S[0, 0].size * g["bytes_per_cell"] == g["dense"][0]["bytes"]


@pytest.mark.parametrize("causal", [False, True])
def test_key_shift_invariance(causal):
    q, k, v = make_qkv(1, 12, 12, 2, 2, 8, "bf16", 1.0, 15)
    qq, kk, vv = _f64(q), _f64(k), _f64(v)
    u = np.linspace(-1.0, 1.5, 8)
    sc = 0.4
    O1, l1 = oracle.attention(qq, kk, vv, sc, causal)
    O2, l2 = oracle.attention(qq, kk + u, vv, sc, causal)
    sigma = float(np.float32(sc))
    assert np.max(np.abs(O1 - O2)) <= 1e-12
    shift = sigma * np.einsum("bihc,c->bhi", qq, u)
    assert np.max(np.abs((l2 - l1) - shift)) <= 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_v_affine(causal):
    q, k, v = make_qkv(2, 10, 14, 4, 2, 6, "bf16", 1.0, 16)
    qq, kk, vv = _f64(q), _f64(k), _f64(v)
    O1, _ = oracle.attention(qq, kk, vv, 0.3, causal)
    O2, _ = oracle.attention(qq, kk, -2.5 * vv + 0.75, 0.3, causal)
    if causal:  # rows with no visible key stay 0 (empty sum), the rest are affine
        Nq, Nk = 10, 14
        assert Nk >= Nq  # every row sees a key here
    assert np.max(np.abs(O2 - (-2.5 * O1 + 0.75))) <= 1e-12


def test_key_permutation_noncausal():
    q, k, v = make_qkv(1, 9, 21, 2, 1, 8, "bf16", 1.0, 17)
    perm = torch.randperm(21, generator=torch.Generator().manual_seed(3))
    O1, l1 = oracle.attention(q, k, v, 0.35, False)
    O2, l2 = oracle.attention(q, k[:, perm], v[:, perm], 0.35, False)
    assert np.max(np.abs(O1 - O2)) <= 1e-12
    assert np.max(np.abs(l1 - l2)) <= 1e-12


@pytest.mark.parametrize("Hq,Hkv", [(8, 2), (6, 3), (4, 1)])
def test_gqa_equals_repeated_mha(Hq, Hkv):
    q, k, v = make_qkv(2, 7, 9, Hq, Hkv, 4, "bf16", 1.0, 18)
    G = Hq // Hkv
    O1, l1 = oracle.attention(q, k, v, 0.5, True)
    O2, l2 = oracle.attention(q, k.repeat_interleave(G, dim=2), v.repeat_interleave(G, dim=2), 0.5, True)
    assert np.array_equal(O1, O2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Hq,Hkv,N,d", [(4, 4, 64, 64), (8, 2, 37, 16), (4, 1, 128, 64)])
def test_matches_torch_sdpa_cpu_fp64(causal, Hq, Hkv, N, d):
    q, k, v = make_qkv(2, N, N, Hq, Hkv, d, "fp16", 1.0, 19)
    sc = 1.0 / math.sqrt(d)
    O, _ = oracle.attention(q, k, v, sc, causal)
    sigma = float(np.float32(sc))
    ref = F.scaled_dot_product_attention(
        q.double().transpose(1, 2), k.double().transpose(1, 2), v.double().transpose(1, 2),
        is_causal=causal, scale=sigma, enable_gqa=(Hq != Hkv)).transpose(1, 2).numpy()
    assert np.max(np.abs(O - ref)) <= 1e-12


def test_pages_sdpa_example_shape():
    # tokenwerk.de page, section "Ein begrenztes SDPA-Beispiel lesen": q of
    # shape (1, 4, 128, 64) in [B, H, N, d], k and v like q, no mask, default
    # scale 1/sqrt(64).  Same computation in this oracle's [B, N, H, d].
    q, k, v = make_qkv(1, 128, 128, 4, 4, 64, "fp16", 1.0, 20)
    O, _ = oracle.attention(q, k, v, 1.0 / 8.0, False)
    ref = F.scaled_dot_product_attention(q.double().transpose(1, 2), k.double().transpose(1, 2),
                                         v.double().transpose(1, 2), dropout_p=0.0)
    assert tuple(ref.shape) == (1, 4, 128, 64)
    assert np.max(np.abs(O - ref.transpose(1, 2).numpy())) <= 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_rows_and_slabs_are_the_same_definition(causal):
    q, k, v = make_qkv(2, 50, 50, 4, 2, 8, "bf16", 1.0, 21)
    O, lse = oracle.attention(q, k, v, 0.3, causal)
    O7, lse7 = oracle.attention(q, k, v, 0.3, causal, slab_rows=7)
    # Same values; BLAS may block a 7-row and a 50-row product differently,
    # so allow last-bit differences.
    assert np.max(np.abs(O - O7)) <= 1e-14 and np.max(np.abs(lse - lse7)) <= 1e-14
    rows = [0, 1, 13, 49]
    Or, lr = oracle.attention_rows(q, k, v, 0.3, causal, 1, 3, rows)
    assert np.max(np.abs(Or - O[1, rows, 3])) <= 1e-15
    assert np.max(np.abs(lr - lse[1, 3, rows])) <= 1e-15


def test_fully_masked_rows():
    q, k, v = make_qkv(1, 6, 2, 1, 1, 4, "bf16", 1.0, 22)
    O, lse = oracle.attention(q, k, v, 0.5, True)
    # j <= i + (2 - 6): rows 0..3 see nothing, row 4 sees key 0, row 5 keys 0..1
    assert np.all(O[0, :4] == 0.0) and np.all(lse[0, 0, :4] == -np.inf)
    assert np.array_equal(O[0, 4, 0], _f64(v)[0, 0, 0])


# ---------------------------------------------------------------------------
# Mutation checks: plant a mistake in the oracle and show that a pin fails.
# ---------------------------------------------------------------------------

def _pins_pass():
    """A compact run of the brute-force and closed-form pins; True if all hold."""
    try:
        for shape in TINY:
            test_oracle_matches_brute_force(shape, None)
        test_causal_row0_is_v0(8)
        test_gqa_equals_repeated_mha(8, 2)
    except AssertionError:
        return False
    return True


def test_pins_pass_unmutated():
    assert _pins_pass()


def test_mutation_wrong_gqa_grouping(monkeypatch):
    monkeypatch.setattr(oa, "kv_head_of", lambda h, Hq, Hkv: h % Hkv)
    assert not _pins_pass()


def test_mutation_causal_off_by_one(monkeypatch):
    real = oa.allowed_keys
    monkeypatch.setattr(oa, "allowed_keys", lambda i, Nq, Nk, c: max(0, real(i, Nq, Nk, c) - 1) if c else Nk)
    assert not _pins_pass()


def test_mutation_top_left_causal(monkeypatch):
    monkeypatch.setattr(oa, "allowed_keys", lambda i, Nq, Nk, c: min(Nk, i + 1) if c else Nk)
    assert not _pins_pass()


def test_mutation_transposed_value_rows(monkeypatch):
    real = oa._rows_of_one_head

    def wrong(qh, kg, vg, sigma, rows, Nq, Nk, causal, want_p, *mods):
        return real(qh, kg, vg[::-1].copy(), sigma, rows, Nq, Nk, causal, want_p, *mods)

    monkeypatch.setattr(oa, "_rows_of_one_head", wrong)
    assert not _pins_pass()


def test_mutation_dropped_scale(monkeypatch):
    real = oa._rows_of_one_head

    def wrong(qh, kg, vg, sigma, rows, Nq, Nk, causal, want_p, *mods):
        return real(qh, kg, vg, 1.0, rows, Nq, Nk, causal, want_p, *mods)

    monkeypatch.setattr(oa, "_rows_of_one_head", wrong)
    assert not _pins_pass()
