"""GPU parity of the backward pass: the HIP kernels (through the C ABI)
against the fp64 backward oracle.

Criterion: the test rule of the hysenlabs.com page (section "Tests,
BSD-3-Clause und Zitierpraxis"): gradients must match a reference within a
numerical tolerance such that the maximum error is at most twice that of a
baseline.  The reference is the fp64 oracle; the baseline is a plain
low-precision backward on the CPU that receives the same inputs as the
kernels -- q, k, v, dout and the forward's rounded out (from which D is
formed) -- and computes in fp32, rounding P and dS to the element type
before their products and every output: the error any bf16/fp16 backward
carries given those inputs.  The mean error gets the same factor.  delta (sum of dout * out) is
compared with the oracle's D within the error that rounding out to the
element type allows.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from attn_workloads import WORKLOADS, make_qkv, make_workload

pytestmark = pytest.mark.gpu


def gpu_fwd_bwd(q, k, v, do, scale, causal):
    from exact_tiled_attention_35_amd import attn_bwd, attn_fwd

    qc, kc, vc, dc = (x.cuda() for x in (q, k, v, do))
    out, lse = attn_fwd(qc, kc, vc, scale, causal)
    dq, dk, dv, delta = attn_bwd(qc, kc, vc, out, dc, lse, scale, causal)
    torch.cuda.synchronize()
    return [x.cpu() for x in (dq, dk, dv, delta, out, lse)]


def lowp_backward(q, k, v, do, out, scale, causal):
    """The low-precision yardstick (CPU, fp32, [B, N, H, d] in and out);
    ``out`` is the forward output the backward receives."""
    dt = q.dtype
    B, Nq, Hq, d = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    G = Hq // Hkv
    qf, dof = q.float().transpose(1, 2), do.float().transpose(1, 2)
    kf = k.float().transpose(1, 2).repeat_interleave(G, 1)
    vf = v.float().transpose(1, 2).repeat_interleave(G, 1)
    sc = float(np.float32(scale))
    s = (qf @ kf.transpose(-1, -2).contiguous()) * sc
    vis = torch.ones(Nq, Nk, dtype=torch.bool)
    if causal:
        vis = torch.arange(Nk)[None, :] <= torch.arange(Nq)[:, None] + (Nk - Nq)
    s = s.masked_fill(~vis, float("-inf"))
    p = torch.softmax(s, -1).nan_to_num(0.0)
    D = (dof * out.float().transpose(1, 2)).sum(-1, keepdim=True)
    dv = p.to(dt).float().transpose(-1, -2) @ dof
    dp = dof @ vf.transpose(-1, -2).contiguous()
    ds = (p * (dp - D)).to(dt).float()
    dq = sc * (ds @ kf)
    dk = sc * (ds.transpose(-1, -2).contiguous() @ qf)
    dk = dk.reshape(B, Hkv, G, Nk, d).sum(2)
    dv = dv.reshape(B, Hkv, G, Nk, d).sum(2)
    return [x.to(dt).transpose(1, 2).double().numpy() for x in (dq, dk, dv)]


def check_grads(got, want, base, what):
    """Max and mean error at most twice the baseline's (both vs the oracle)."""
    out = []
    for name, g, w, b in zip(("dq", "dk", "dv"), got, want, base):
        g = g.double().numpy()
        assert np.all(np.isfinite(g)), f"{what} {name} not finite"
        err, berr = np.abs(g - w), np.abs(b - w)
        assert err.max() <= 2.0 * berr.max() + 1e-6, \
            f"{what} {name}: max {err.max():.3e} vs baseline {berr.max():.3e}"
        assert err.mean() <= 2.0 * berr.mean() + 1e-7, \
            f"{what} {name}: mean {err.mean():.3e} vs baseline {berr.mean():.3e}"
        out.append((name, float(err.max()), float(berr.max())))
    return out


def check_delta(delta, D, do, out):
    # delta is computed from the kernel's rounded out, whose error is at most
    # about one ulp of |O| (half an ulp of rounding plus the forward's own
    # error): |delta - D| <= sum_c |dO_c| (|O_c| ulp + 1e-5).
    ulp = 2.0 ** -7 if out.dtype == torch.bfloat16 else 2.0 ** -10
    per = np.abs(do.double().numpy()) * (np.abs(out.double().numpy()) * ulp + 1e-5)
    bound = per.sum(-1).transpose(0, 2, 1) + 1e-5
    assert np.all(np.abs(delta.double().numpy() - D) <= bound)


SMALL = [  # (B, Hq, Hkv, Nq, Nk, d, dtype, causal)
    (1, 1, 1, 1, 1, 64, "bf16", False),
    (1, 2, 1, 3, 2, 128, "bf16", True),
    (1, 1, 1, 17, 17, 128, "bf16", True),
    (2, 4, 2, 63, 65, 128, "bf16", False),
    (1, 4, 4, 64, 64, 64, "fp16", True),
    (1, 2, 1, 65, 127, 128, "bf16", True),
    (1, 8, 1, 127, 128, 128, "bf16", False),
    (1, 2, 2, 128, 129, 256, "fp16", True),
    (1, 2, 2, 129, 128, 256, "bf16", False),
    (2, 8, 2, 255, 255, 64, "bf16", True),
    (1, 2, 1, 600, 600, 128, "bf16", True),
    (1, 4, 2, 300, 1000, 128, "bf16", True),
    (1, 2, 2, 1000, 300, 64, "bf16", True),
    (1, 2, 2, 257, 513, 256, "bf16", True),
    (3, 6, 3, 129, 200, 64, "fp16", False),
    (1, 4, 1, 511, 511, 128, "fp16", True),
    # non-causal d = 128 (the dK/dV kernel's 256-key workgroups): key counts
    # across and around 256, ragged tails, GQA
    (1, 4, 2, 300, 257, 128, "bf16", False),
    (2, 2, 1, 200, 600, 128, "fp16", False),
    (1, 4, 4, 96, 513, 128, "bf16", False),
    (1, 2, 2, 33, 256, 128, "bf16", False),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "B%dH%d-%dN%dx%dd%d%s%s" % (
    c[0], c[1], c[2], c[3], c[4], c[5], c[6], "c" if c[7] else ""))
def test_backward_small_grid(case):
    B, Hq, Hkv, Nq, Nk, d, dt, causal = case
    seed = 600 + SMALL.index(case)
    q, k, v = make_qkv(B, Nq, Nk, Hq, Hkv, d, dt, 1.0, seed)
    do = make_qkv(B, Nq, Nq, Hq, Hq, d, dt, 1.0, seed + 1000)[0]
    scale = 1.0 / math.sqrt(d)
    dq, dk, dv, delta, out, _ = gpu_fwd_bwd(q, k, v, do, scale, causal)
    want = oracle.attention_backward(q, k, v, do, scale, causal)
    base = lowp_backward(q, k, v, do, out, scale, causal)
    check_grads((dq, dk, dv), want[:3], base, str(case))
    check_delta(delta, want[3], do, out)


@pytest.mark.parametrize("scale", [-0.3, 0.0, 0.5])
def test_backward_unusual_scales(scale):
    q, k, v = make_qkv(1, 200, 200, 2, 1, 128, "bf16", 1.0, 700)
    do = make_qkv(1, 200, 200, 2, 2, 128, "bf16", 1.0, 701)[0]
    for causal in (False, True):
        dq, dk, dv, _, out, _ = gpu_fwd_bwd(q, k, v, do, scale, causal)
        want = oracle.attention_backward(q, k, v, do, scale, causal)
        check_grads((dq, dk, dv), want[:3], lowp_backward(q, k, v, do, out, scale, causal),
                    f"scale {scale} causal {causal}")


def test_backward_rows_without_keys_and_no_queries():
    # Causal with Nq > Nk: the first Nq - Nk rows see no key; their dq is 0.
    q, k, v = make_qkv(1, 150, 70, 2, 2, 128, "bf16", 1.0, 702)
    do = make_qkv(1, 150, 150, 2, 2, 128, "bf16", 1.0, 703)[0]
    dq, dk, dv, delta, out, lse = gpu_fwd_bwd(q, k, v, do, 0.1, True)
    assert torch.all(dq[:, :80] == 0)
    want = oracle.attention_backward(q, k, v, do, 0.1, True)
    check_grads((dq, dk, dv), want[:3], lowp_backward(q, k, v, do, out, 0.1, True), "empty rows")
    # Nq == 0: dk and dv are zero, nothing else is touched.
    from exact_tiled_attention_35_amd import attn_bwd_ptr, _lib
    kc = torch.randn(1, 64, 2, 128, device="cuda").to(torch.bfloat16)
    dk0 = torch.full_like(kc, 7.0)
    dv0 = torch.full_like(kc, 7.0)
    code = attn_bwd_ptr(0, kc.data_ptr(), kc.data_ptr(), 0, 0, 0, 0, dk0.data_ptr(), dv0.data_ptr(),
                        0, 1, 2, 2, 0, 64, 128, 0.1, True, _lib.ATTN_DTYPE_BF16,
                        torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert code == 0
    assert torch.all(dk0 == 0) and torch.all(dv0 == 0)


@pytest.mark.parametrize("Nq,Nk,causal", [(300, 300, True), (333, 190, True), (190, 333, False)])
def test_backward_large_logits(Nq, Nk, causal):
    # Inputs with sigma 8 give scaled scores with a spread of ~64: hidden
    # (causal or past-the-end) pairs then lie up to ~200 above the row's
    # logsumexp, so their exponential overflows fp32 and must be dropped
    # before it reaches dS, dK or dV.
    q, k, v = make_qkv(1, Nq, Nk, 2, 1, 128, "bf16", 8.0, 710)
    do = make_qkv(1, Nq, Nq, 2, 2, 128, "bf16", 1.0, 711)[0]
    scale = 1.0 / math.sqrt(128)
    dq, dk, dv, delta, out, _ = gpu_fwd_bwd(q, k, v, do, scale, causal)
    assert all(torch.isfinite(x.float()).all() for x in (dq, dk, dv, delta))
    want = oracle.attention_backward(q, k, v, do, scale, causal)
    check_grads((dq, dk, dv), want[:3], lowp_backward(q, k, v, do, out, scale, causal),
                f"large logits {Nq}x{Nk} causal {causal}")
    check_delta(delta, want[3], do, out)


def test_backward_invariants():
    q, k, v = make_qkv(1, 300, 300, 4, 2, 128, "bf16", 1.0, 704)
    do = make_qkv(1, 300, 300, 4, 4, 128, "bf16", 1.0, 705)[0]
    dq, dk, dv, delta, out, lse = gpu_fwd_bwd(q, k, v, do, 0.088, False)
    # Key gradients of a head sum to ~0; value gradients sum to the dout rows.
    scale_k = dk.double().abs().sum(1).max()
    assert dk.double().sum(1).abs().max() <= 2e-2 * scale_k
    want_v = do.double().reshape(1, 300, 2, 2, 128).sum((1, 3))
    assert (dv.double().sum(1) - want_v).abs().max() <= 2e-2 * want_v.abs().max()
    # Zero dout: exactly zero gradients.
    z = gpu_fwd_bwd(q, k, v, torch.zeros_like(do), 0.088, True)
    assert all(torch.all(x == 0) for x in z[:4])
    # Constant V: dq and dk vanish (up to fp32 rounding of dP - D).
    vc = torch.full_like(v, 0.25)
    r = gpu_fwd_bwd(q, k, vc, do, 0.088, True)
    assert r[0].double().abs().max() <= 1e-3 and r[1].double().abs().max() <= 1e-3


def test_backward_is_deterministic():
    q, k, v = make_qkv(2, 400, 400, 8, 2, 128, "bf16", 1.0, 706)
    do = make_qkv(2, 400, 400, 8, 8, 128, "bf16", 1.0, 707)[0]
    a = gpu_fwd_bwd(q, k, v, do, 0.088, True)
    b = gpu_fwd_bwd(q, k, v, do, 0.088, True)
    assert all(torch.equal(x, y) for x, y in zip(a, b))


def test_autograd_wrapper_matches_entry_points():
    from exact_tiled_attention_35_amd import attention, attn_bwd, attn_fwd

    q, k, v = (x.cuda() for x in make_qkv(1, 130, 130, 4, 2, 64, "bf16", 1.0, 708))
    do = make_qkv(1, 130, 130, 4, 4, 64, "bf16", 1.0, 709)[0].cuda()
    qa, ka, va = (x.clone().requires_grad_(True) for x in (q, k, v))
    o = attention(qa, ka, va, None, True)
    o.backward(do)
    out, lse = attn_fwd(q, k, v, None, True)
    dq, dk, dv, _ = attn_bwd(q, k, v, out, do, lse, None, True)
    assert torch.equal(o.detach(), out)
    assert torch.equal(qa.grad, dq) and torch.equal(ka.grad, dk) and torch.equal(va.grad, dv)


@pytest.mark.parametrize("name", ["mha_b4_h16_n4096_d128_bf16", "causal_mha_b2_h32_n8192_d128_bf16"])
def test_backward_workload_heads(name):
    # Full-size gradients for a few whole KV groups (every query head that
    # reads the KV head, every row): the oracle evaluates just those slices.
    w = WORKLOADS[name]
    q, k, v = make_workload(w)
    do = make_qkv(w.B, w.Nq, w.Nq, w.Hq, w.Hq, w.d, w.dtype, w.sigma, w.seed + 100)[0]
    dq, dk, dv, delta, out, _ = gpu_fwd_bwd(q, k, v, do, w.scale, w.causal)
    G = w.Hq // w.Hkv
    worst = []
    for (b, g) in sorted({(0, 0), (w.B - 1, w.Hkv - 1)}):
        hs = slice(g * G, (g + 1) * G)
        sl = lambda x, h: x[b:b + 1, :, h]
        qs, ks, vs, ds = sl(q, hs), sl(k, slice(g, g + 1)), sl(v, slice(g, g + 1)), sl(do, hs)
        want = oracle.attention_backward(qs, ks, vs, ds, w.scale, w.causal)
        base = lowp_backward(qs, ks, vs, ds, sl(out, hs), w.scale, w.causal)
        got = (sl(dq, hs), sl(dk, slice(g, g + 1)), sl(dv, slice(g, g + 1)))
        worst += check_grads(got, want[:3], base, f"{name} b{b} g{g}")
    print(f"[parity-bwd] {name}: " + ", ".join(f"{n} {e:.2e} (base {b_:.2e})" for n, e, b_ in worst),
          flush=True)
