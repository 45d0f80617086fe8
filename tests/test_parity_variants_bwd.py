"""GPU parity of the backward with score variants (attn_bwd_ext: sliding
window, ALiBi, softcap) against the fp64 oracle (attention_backward with the
same variants), with the backward's criterion: max and mean error at most
twice those of a plain low-precision backward that computes the same
variants in fp32 from the same inputs (P and dS rounded to the element type
before their products)."""

import numpy as np
import pytest
import torch

import oracle
from attn_workloads import WORKLOADS, make_qkv, make_workload
from test_parity_bwd import check_delta, check_grads

pytestmark = pytest.mark.gpu


def slopes_for(Hq):
    return torch.tensor([2.0 ** (-8.0 * (h + 1) / Hq) for h in range(Hq)], dtype=torch.float32)


def lowp_backward_variants(q, k, v, do, out, scale, causal, window, slopes, cap):
    dt = q.dtype
    B, Nq, Hq, d = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    G = Hq // Hkv
    qf, dof = q.float().transpose(1, 2), do.float().transpose(1, 2)
    kf = k.float().transpose(1, 2).repeat_interleave(G, 1)
    vf = v.float().transpose(1, 2).repeat_interleave(G, 1)
    sc = float(np.float32(scale))
    s = (qf @ kf.transpose(-1, -2).contiguous()) * sc
    gcap = torch.ones_like(s)
    if cap > 0:
        th = torch.tanh(s / cap)
        s, gcap = cap * th, 1 - th * th
    dist = (torch.arange(Nq)[:, None] + (Nk - Nq)) - torch.arange(Nk)[None, :]
    if slopes is not None:
        s = s - slopes.float()[None, :, None, None] * dist.abs().float()
    vis = torch.ones(Nq, Nk, dtype=torch.bool)
    if causal:
        vis &= dist >= 0
    if window[0] >= 0:
        vis &= dist <= window[0]
    if window[1] >= 0:
        vis &= -dist <= window[1]
    s = s.masked_fill(~vis, float("-inf"))
    p = torch.softmax(s, -1).nan_to_num(0.0)
    D = (dof * out.float().transpose(1, 2)).sum(-1, keepdim=True)
    dv = p.to(dt).float().transpose(-1, -2) @ dof
    dp = dof @ vf.transpose(-1, -2).contiguous()
    ds = (p * (dp - D) * gcap).to(dt).float()
    dq = sc * (ds @ kf)
    dk = sc * (ds.transpose(-1, -2).contiguous() @ qf)
    dk = dk.reshape(B, Hkv, G, Nk, d).sum(2)
    dv = dv.reshape(B, Hkv, G, Nk, d).sum(2)
    return [x.to(dt).transpose(1, 2).double().numpy() for x in (dq, dk, dv)]


def gpu_fwd_bwd(q, k, v, do, scale, causal, window, slopes, cap):
    from exact_tiled_attention_35_amd import attn_bwd, attn_fwd

    qc, kc, vc, dc = (x.cuda() for x in (q, k, v, do))
    sl = slopes.cuda() if slopes is not None else None
    out, lse = attn_fwd(qc, kc, vc, scale, causal, window=window, alibi_slopes=sl, softcap=cap)
    dq, dk, dv, delta = attn_bwd(qc, kc, vc, out, dc, lse, scale, causal, window=window,
                                 alibi_slopes=sl, softcap=cap)
    torch.cuda.synchronize()
    return [x.cpu() for x in (dq, dk, dv, delta, out, lse)]


# (B, Hq, Hkv, Nq, Nk, d, dtype, causal, window, alibi, softcap)
CASES = [
    (1, 4, 2, 300, 300, 128, "bf16", True, (100, 0), False, 0.0),
    (1, 2, 2, 257, 400, 64, "fp16", False, (64, 64), False, 0.0),
    (2, 4, 1, 200, 200, 128, "bf16", False, (-1, -1), True, 0.0),
    (1, 2, 2, 300, 260, 128, "bf16", True, (-1, -1), False, 5.0),
    (1, 4, 2, 129, 500, 256, "bf16", False, (50, 10), True, 20.0),
    (1, 2, 1, 400, 400, 64, "bf16", True, (255, -1), True, 30.0),
    # every variant kind (window only, softcap, ALiBi, both) at every head
    # dim on tiles cut by a window, a ragged end or empty rows
    (1, 2, 1, 190, 333, 256, "fp16", True, (80, 20), False, 0.0),
    (2, 2, 2, 333, 190, 64, "bf16", False, (40, 70), False, 10.0),
    (1, 2, 2, 160, 160, 256, "fp16", True, (-1, -1), False, 15.0),
    (1, 2, 1, 260, 380, 128, "bf16", False, (60, 60), False, 8.0),
    (1, 4, 4, 250, 300, 64, "fp16", True, (100, 0), True, 0.0),
    (1, 2, 1, 300, 200, 256, "bf16", False, (-1, 30), True, 0.0),
    (1, 2, 2, 500, 300, 128, "bf16", True, (150, -1), True, 0.0),
    (1, 4, 2, 350, 350, 128, "fp16", False, (90, 40), True, 25.0),
]


@pytest.mark.parametrize("ci", range(len(CASES)))
def test_variant_backward_against_oracle(ci):
    B, Hq, Hkv, Nq, Nk, d, dt, causal, window, alibi, cap = CASES[ci]
    q, k, v = make_qkv(B, Nq, Nk, Hq, Hkv, d, dt, 1.0, 1500 + ci)
    do = make_qkv(B, Nq, Nk, Hq, Hkv, d, dt, 1.0, 1550 + ci)[0]
    slopes = slopes_for(Hq) if alibi else None
    scale = 1.0 / np.sqrt(d)
    dq, dk, dv, delta, out, lse = gpu_fwd_bwd(q, k, v, do, scale, causal, window, slopes, cap)
    want = oracle.attention_backward(q, k, v, do, scale, causal, window=window,
                                     alibi_slopes=slopes.numpy() if alibi else None, softcap=cap)
    base = lowp_backward_variants(q, k, v, do, out, scale, causal, window, slopes, cap)
    check_grads((dq, dk, dv), want[:3], base, f"case {ci}")
    check_delta(delta, want[3], do, out)


@pytest.mark.parametrize("cap", [0.0, 200.0])
def test_variant_backward_large_logits(cap):
    # sigma 8 inputs: hidden pairs of the window's edge tiles overflow the
    # exponential; the mask pass must drop them (softcap 200 barely caps).
    B, Hq, Hkv, Nq, Nk, d = 1, 2, 1, 333, 300, 128
    q, k, v = make_qkv(B, Nq, Nk, Hq, Hkv, d, "bf16", 8.0, 1580)
    do = make_qkv(B, Nq, Nk, Hq, Hkv, d, "bf16", 1.0, 1581)[0]
    slopes, window, scale = slopes_for(Hq), (90, 10), 1.0 / np.sqrt(d)
    dq, dk, dv, delta, out, lse = gpu_fwd_bwd(q, k, v, do, scale, True, window, slopes, cap)
    assert all(torch.isfinite(x.float()).all() for x in (dq, dk, dv, delta))
    want = oracle.attention_backward(q, k, v, do, scale, True, window=window,
                                     alibi_slopes=slopes.numpy(), softcap=cap)
    base = lowp_backward_variants(q, k, v, do, out, scale, True, window, slopes, cap)
    check_grads((dq, dk, dv), want[:3], base, f"large logits cap {cap}")
    check_delta(delta, want[3], do, out)


def test_autograd_wrapper_with_variants_matches_entry_points():
    from exact_tiled_attention_35_amd import attention, attn_bwd, attn_fwd

    q, k, v = (x.cuda() for x in make_qkv(1, 200, 230, 4, 2, 128, "bf16", 1.0, 1595))
    do = make_qkv(1, 200, 230, 4, 2, 128, "bf16", 1.0, 1596)[0].cuda()
    sl = slopes_for(4).cuda()
    kw = dict(window=(64, 8), alibi_slopes=sl, softcap=20.0)
    qa, ka, va = (x.clone().requires_grad_(True) for x in (q, k, v))
    o = attention(qa, ka, va, None, True, **kw)
    o.backward(do)
    out, lse = attn_fwd(q, k, v, None, True, **kw)
    dq, dk, dv, _ = attn_bwd(q, k, v, out, do, lse, None, True, **kw)
    assert torch.equal(o.detach(), out)
    assert torch.equal(qa.grad, dq) and torch.equal(ka.grad, dk) and torch.equal(va.grad, dv)


def test_variant_backward_is_deterministic():
    B, Hq, Hkv, Nq, Nk, d, dt, causal, window, alibi, cap = CASES[4]
    q, k, v = make_qkv(B, Nq, Nk, Hq, Hkv, d, dt, 1.0, 1590)
    do = make_qkv(B, Nq, Nk, Hq, Hkv, d, dt, 1.0, 1591)[0]
    a = gpu_fwd_bwd(q, k, v, do, 0.1, causal, window, slopes_for(Hq), cap)
    b = gpu_fwd_bwd(q, k, v, do, 0.1, causal, window, slopes_for(Hq), cap)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_headline_shape_softcap_and_alibi_full_size_head():
    """The headline shape with softcap 30 and ALiBi (the benched forward
    variants) at full size; one KV group's gradients against the oracle."""
    w = WORKLOADS["mha_b4_h16_n4096_d128_bf16"]
    q, k, v = make_workload(w)
    do = make_qkv(w.B, w.Nq, w.Nk, w.Hq, w.Hkv, w.d, w.dtype, w.sigma, w.seed + 100)[0]
    slopes = slopes_for(w.Hq)
    dq, dk, dv, delta, out, lse = gpu_fwd_bwd(q, k, v, do, w.scale, w.causal, (-1, -1), slopes, 30.0)
    b, h = 1, 5
    sl = lambda x: x[b:b + 1, :, h:h + 1]  # noqa: E731
    want = oracle.attention_backward(sl(q), sl(k), sl(v), sl(do), w.scale, w.causal,
                                     alibi_slopes=slopes.numpy()[h:h + 1], softcap=30.0)
    base = lowp_backward_variants(sl(q), sl(k), sl(v), sl(do), sl(out), w.scale, w.causal, (-1, -1),
                                  slopes[h:h + 1], 30.0)
    check_grads((sl(dq), sl(dk), sl(dv)), want[:3], base, "headline softcap+alibi")


def test_binding_sends_every_window_to_the_checked_entry_point():
    # A window bound below -1 is an error of the C ABI; the binding must not
    # take (-2, -2) for "no window" and run the plain kernel.
    from exact_tiled_attention_35_amd import attn_bwd, attn_fwd
    from exact_tiled_attention_35_amd.attention import AttnError

    q, k, v = (t.cuda() for t in make_qkv(1, 64, 64, 2, 2, 64, "bf16", 1.0, 611))
    for win in ((-2, -2), (-2, -1), (-1, -5)):
        with pytest.raises(AttnError) as e:
            attn_fwd(q, k, v, 0.125, False, window=win)
        assert "BAD_ARGUMENT" in str(e.value)
    out, lse = attn_fwd(q, k, v, 0.125, False)
    with pytest.raises(AttnError):
        attn_bwd(q, k, v, out, torch.ones_like(out), lse, 0.125, False, window=(-2, -2))


def test_autograd_detects_slopes_changed_in_place():
    # The ALiBi slopes are saved for the backward like the tensors: changing
    # them in place between forward and backward is an error, not silently
    # wrong gradients.
    from exact_tiled_attention_35_amd import attention

    q, k, v = (t.cuda().requires_grad_() for t in make_qkv(1, 64, 64, 2, 2, 64, "bf16", 1.0, 612))
    slopes = slopes_for(2).cuda()
    out = attention(q, k, v, 0.125, True, alibi_slopes=slopes)
    slopes.mul_(2.0)
    with pytest.raises(RuntimeError, match="modified by an inplace operation"):
        out.float().sum().backward()
