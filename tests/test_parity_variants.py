"""GPU parity of the score variants (attn_fwd_ext: sliding window, ALiBi,
softcap) against the fp64 oracle, at the forward's tolerances (mean-abs
1e-3, lse 1e-3; rows with no kept key exactly 0 / -inf) and a max-abs error
of 1e-2 or, where a window leaves rows with a handful of keys so that the
output's own rounding approaches 1e-2, at most twice that of a plain
low-precision attention with the same variants (the test rule of the
hysenlabs.com page, section "Tests, BSD-3-Clause und Zitierpraxis")."""

import math

import numpy as np
import pytest
import torch

import oracle
from attn_workloads import make_qkv

pytestmark = pytest.mark.gpu

MAX_ABS, MEAN_ABS, LSE_ABS = 1e-2, 1e-3, 1e-3


def slopes_for(Hq):
    return torch.tensor([2.0 ** (-8.0 * (h + 1) / Hq) for h in range(Hq)], dtype=torch.float32)


def lowp_variant(q, k, v, scale, causal, window, slopes, cap):
    """Plain low-precision attention with the variants (CPU, fp32; P and the
    output rounded to the element type)."""
    dt = q.dtype
    B, Nq, Hq, d = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    G = Hq // Hkv
    qf = q.float().transpose(1, 2)
    kf = k.float().transpose(1, 2).repeat_interleave(G, 1)
    vf = v.float().transpose(1, 2).repeat_interleave(G, 1)
    t = (qf @ kf.transpose(-1, -2).contiguous()) * float(np.float32(scale))
    if cap > 0:
        t = cap * torch.tanh(t / cap)
    i = torch.arange(Nq)[:, None]
    j = torch.arange(Nk)[None, :]
    dist = i + (Nk - Nq) - j
    if slopes is not None:
        t = t - slopes.float()[:, None, None] * dist.abs().float()
    vis = torch.ones(Nq, Nk, dtype=torch.bool)
    if causal:
        vis &= dist >= 0
    if window[0] >= 0:
        vis &= dist <= window[0]
    if window[1] >= 0:
        vis &= -dist <= window[1]
    p = torch.softmax(t.masked_fill(~vis, float("-inf")), -1).nan_to_num(0.0)
    return (p.to(dt).float() @ vf).to(dt).transpose(1, 2).double().numpy()


def check(case, window, use_alibi, cap, seed, scale=None):
    from exact_tiled_attention_35_amd import attn_fwd

    B, Hq, Hkv, Nq, Nk, d, dt, causal = case
    q, k, v = make_qkv(B, Nq, Nk, Hq, Hkv, d, dt, 1.0, seed)
    sl = slopes_for(Hq) if use_alibi else None
    sc = 1.0 / math.sqrt(d) if scale is None else scale
    out, lse = attn_fwd(q.cuda(), k.cuda(), v.cuda(), sc, causal, window=window,
                        alibi_slopes=sl.cuda() if sl is not None else None, softcap=cap)
    torch.cuda.synchronize()
    O, L = oracle.attention(q, k, v, sc, causal, window=window,
                            alibi_slopes=sl.numpy() if sl is not None else None, softcap=cap)
    o, lg = out.cpu().double().numpy(), lse.cpu().double().numpy()
    err = np.abs(o - O)
    assert err.mean() <= MEAN_ABS, err.mean()
    if err.max() > MAX_ABS:
        base = np.abs(lowp_variant(q, k, v, sc, causal, window, sl, cap) - O).max()
        assert err.max() <= 2.0 * base, (err.max(), base)
    fin = np.isfinite(L)
    assert np.array_equal(np.isfinite(lg), fin)
    assert np.all(lg[~fin] == -np.inf)
    if fin.any():
        assert np.abs(lg[fin] - L[fin]).max() <= LSE_ABS
    empty = np.broadcast_to((~fin).transpose(0, 2, 1)[..., None], o.shape)
    assert np.all(o[empty] == 0)
    return float(err.max())


SHAPES = [  # (B, Hq, Hkv, Nq, Nk, d, dtype, causal)
    (1, 4, 2, 300, 300, 128, "bf16", True),
    (2, 2, 2, 200, 333, 64, "fp16", False),
    (1, 2, 1, 257, 190, 256, "bf16", True),
    (1, 8, 8, 129, 513, 128, "bf16", False),
]
VARIANTS = [  # (window, alibi, softcap)
    ((64, -1), False, 0.0),
    ((-1, 0), False, 0.0),
    ((100, 37), False, 0.0),
    ((0, 0), False, 0.0),
    ((-1, -1), True, 0.0),
    ((-1, -1), False, 5.0),
    ((127, 0), True, 20.0),
    ((5, 130), True, 0.0),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda c: "B%dH%d-%dN%dx%dd%d%s%s" % (
    c[0], c[1], c[2], c[3], c[4], c[5], c[6], "c" if c[7] else ""))
@pytest.mark.parametrize("var", VARIANTS, ids=str)
def test_variants_against_oracle(shape, var):
    window, alibi, cap = var
    e = check(shape, window, alibi, cap, 1000 + SHAPES.index(shape) * 10 + VARIANTS.index(var))
    print(f"[parity-variants] {shape} {var}: max-abs {e:.3e}", flush=True)


@pytest.mark.parametrize("scale", [-0.2, 0.0])
def test_window_with_nonpositive_scale(scale):
    check((1, 2, 1, 300, 300, 128, "bf16", True), (70, -1), False, 0.0, 1103, scale=scale)
    check((1, 2, 1, 300, 300, 128, "bf16", False), (70, 20), True, 0.0, 1104, scale=scale)


def test_long_window_interior_tiles():
    # a window much longer than a tile: most tiles are fully inside every
    # row's window and take the unmasked bodies
    check((1, 4, 2, 1100, 1100, 128, "bf16", True), (511, -1), False, 0.0, 1105)
    check((1, 4, 2, 700, 1300, 64, "fp16", False), (300, 200), False, 0.0, 1106)


def test_variants_with_large_scale_and_tight_softcap():
    check((1, 2, 2, 200, 200, 128, "bf16", True), (40, -1), True, 2.0, 1100, scale=0.5)


def test_zero_width_window_returns_the_diagonal_value():
    from exact_tiled_attention_35_amd import attn_fwd

    q, k, v = make_qkv(1, 100, 160, 2, 1, 128, "bf16", 1.0, 1101)
    out, _ = attn_fwd(q.cuda(), k.cuda(), v.cuda(), None, False, window=(0, 0))
    torch.cuda.synchronize()
    assert torch.equal(out.cpu(), v[:, 60:160].expand(1, 100, 2, 128))


def test_inactive_variants_are_attn_fwd_and_no_op_variants_agree():
    from exact_tiled_attention_35_amd import attn_fwd, attn_fwd_ext_ptr, _lib

    q, k, v = (x.cuda() for x in make_qkv(2, 300, 300, 4, 2, 128, "bf16", 1.0, 1102))
    ref, rl = attn_fwd(q, k, v, None, True)
    out, lse = torch.empty_like(q), torch.empty_like(rl)
    code = attn_fwd_ext_ptr(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                            2, 4, 2, 300, 300, 128, 1.0 / math.sqrt(128), True, -1, -1, 0, 0.0,
                            _lib.ATTN_DTYPE_BF16, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert code == 0 and torch.equal(out, ref) and torch.equal(lse, rl)
    # a window wider than the sequence takes the variant kernel and changes nothing
    o2, l2 = attn_fwd(q, k, v, None, True, window=(1000, 1000))
    assert (o2.double() - ref.double()).abs().max() <= 8e-3 and (l2 - rl).abs().max() <= 1e-5


# The variant configurations the bench times, at full size: sampled rows of
# several heads against the oracle (rows near the window edges included).
FULL = [  # (workload, window, alibi, softcap)
    ("causal_gqa_b1_hq64_hkv8_n16384_d128_bf16", (4095, 0), False, 0.0),
    ("causal_mha_b2_h32_n8192_d128_bf16", (1023, 0), False, 0.0),
    ("mha_b4_h16_n4096_d128_bf16", (-1, -1), False, 30.0),
    ("mha_b4_h16_n4096_d128_bf16", (-1, -1), True, 0.0),
]


@pytest.mark.parametrize("cfg", FULL, ids=lambda c: f"{c[0]}-w{c[1][0]}_{c[1][1]}-a{int(c[2])}-c{c[3]:g}")
def test_variant_workloads_full_size(cfg):
    from attn_workloads import WORKLOADS, make_workload
    from exact_tiled_attention_35_amd import attn_fwd

    name, window, alibi, cap = cfg
    w = WORKLOADS[name]
    print(f"[parity-variants] full size {cfg}", flush=True)
    q, k, v = make_workload(w)
    sl = slopes_for(w.Hq) if alibi else None
    out, lse = attn_fwd(q.cuda(), k.cuda(), v.cuda(), w.scale, w.causal, window=window,
                        alibi_slopes=sl.cuda() if sl is not None else None, softcap=cap)
    torch.cuda.synchronize()
    out, lse = out.cpu(), lse.cpu()
    assert torch.isfinite(out).all() and torch.isfinite(lse).all()
    rng = np.random.default_rng(w.seed)
    heads = sorted({(0, 0), (w.B - 1, w.Hq - 1), (0, w.Hq // 2)})
    L = window[0]
    for b, h in heads:
        fixed = {0, 1, 63, 64, 127, 128, w.Nq // 2, w.Nq - 1}
        if L >= 0:
            fixed |= {L - 1, L, L + 1, L + 64, min(w.Nq - 1, 2 * L + 5)}
        rows = sorted(r for r in fixed | {int(x) for x in rng.integers(0, w.Nq, 16)} if 0 <= r < w.Nq)
        O, Lr = oracle.attention_rows(q, k, v, w.scale, w.causal, b, h, rows, window=window,
                                      alibi_slopes=sl.numpy() if sl is not None else None,
                                      softcap=cap)
        err = np.abs(out[b, rows, h].double().numpy() - O)
        assert err.max() <= MAX_ABS and err.mean() <= MEAN_ABS, (b, h, err.max(), err.mean())
        assert np.abs(lse[b, h, rows].double().numpy() - Lr).max() <= LSE_ABS, (b, h)
