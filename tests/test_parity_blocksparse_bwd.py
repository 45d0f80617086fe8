"""GPU parity of the block-sparse backward (attn_bwd_blocksparse) against the
fp64 oracle (attention_backward with the block mask), with the backward's
criterion (the hysenlabs.com page's test rule: max and mean error at most
twice those of a plain low-precision backward given the same inputs, here
with the same mask), and bitwise against attn_bwd where both compute the
same thing with the same tiles."""

import numpy as np
import pytest
import torch

import oracle
from attn_workloads import BLOCK, BLOCKSPARSE_WORKLOADS, WORKLOADS, make_block_mask, make_qkv, make_workload
from test_parity_bwd import check_delta, check_grads

pytestmark = pytest.mark.gpu


def nblocks(n):
    return -(-n // BLOCK)


def element_mask(mask, Hq, Nq, Nk, causal):
    """[B, Hq, Nq, Nk] booleans: the block flags expanded, and causal."""
    m = mask.bool()
    if m.shape[1] == 1:
        m = m.expand(-1, Hq, -1, -1)
    em = m.repeat_interleave(BLOCK, 2)[:, :, :Nq].repeat_interleave(BLOCK, 3)[..., :Nk]
    if causal:
        em = em & (torch.arange(Nk)[None, :] <= torch.arange(Nq)[:, None] + (Nk - Nq))
    return em


def lowp_backward_masked(q, k, v, do, out, scale, vis):
    """The low-precision yardstick of the backward tests, with an element mask."""
    dt = q.dtype
    B, Nq, Hq, d = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    G = Hq // Hkv
    qf, dof = q.float().transpose(1, 2), do.float().transpose(1, 2)
    kf = k.float().transpose(1, 2).repeat_interleave(G, 1)
    vf = v.float().transpose(1, 2).repeat_interleave(G, 1)
    sc = float(np.float32(scale))
    s = (qf @ kf.transpose(-1, -2).contiguous()) * sc
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


def gpu_fwd_bwd(q, k, v, do, mask, scale, causal):
    from exact_tiled_attention_35_amd import attn_bwd_blocksparse, attn_fwd_blocksparse

    qc, kc, vc, dc, mc = (x.cuda() for x in (q, k, v, do, mask))
    out, lse = attn_fwd_blocksparse(qc, kc, vc, mc, scale, causal)
    dq, dk, dv, delta = attn_bwd_blocksparse(qc, kc, vc, out, dc, lse, mc, scale, causal)
    torch.cuda.synchronize()
    return [x.cpu() for x in (dq, dk, dv, delta, out, lse)]


# (B, Hq, Hkv, Nq, Nk, d, dtype, mask heads, density)
CASES = [
    (1, 4, 2, 300, 500, 128, "bf16", 4, 0.5),
    (2, 2, 1, 257, 129, 64, "fp16", 1, 0.6),
    (1, 2, 2, 256, 384, 256, "bf16", 2, 0.5),
    (1, 8, 1, 400, 200, 128, "bf16", 8, 0.7),  # MQA, Nq > Nk
    (1, 4, 4, 700, 900, 64, "bf16", 1, 0.3),
]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("ci", range(len(CASES)))
def test_backward_against_oracle(ci, causal):
    B, Hq, Hkv, Nq, Nk, d, dt, Hm, dens = CASES[ci]
    q, k, v = make_qkv(B, Nq, Nk, Hq, Hkv, d, dt, 1.0, 1100 + ci)
    do = make_qkv(B, Nq, Nk, Hq, Hkv, d, dt, 1.0, 1150 + ci)[0]
    mask = make_block_mask(B, Hm, nblocks(Nq), nblocks(Nk), dens, 1170 + ci)
    mask[0, 0, 0, :] = 0  # a query block that keeps no key
    scale = 1.0 / np.sqrt(d)
    dq, dk, dv, delta, out, lse = gpu_fwd_bwd(q, k, v, do, mask, scale, causal)
    want = oracle.attention_backward(q, k, v, do, scale, causal, block_mask=mask)
    vis = element_mask(mask, Hq, Nq, Nk, causal)
    base = lowp_backward_masked(q, k, v, do, out, scale, vis)
    check_grads((dq, dk, dv), want[:3], base, f"case {ci} causal {causal}")
    check_delta(delta, want[3], do, out)
    assert (dq[0, :BLOCK, 0] == 0).all()


@pytest.mark.parametrize("causal", [False, True])
def test_all_ones_is_bitwise_attn_bwd(causal):
    from exact_tiled_attention_35_amd import attn_bwd, attn_fwd

    # Both backward calls take the block-sparse forward's out and lse (the
    # plain forward equals it bit for bit only when causal: not causal it
    # walks 128-key tiles where the block-sparse forward walks 64-key ones);
    # the plain forward is still checked against them to rounding.
    B, Hq, Hkv, Nq, Nk, d = 2, 24, 6, 320, 448, 128
    q, k, v = make_qkv(B, Nq, Nk, Hq, Hkv, d, "bf16", 1.0, 1180)
    do = make_qkv(B, Nq, Nk, Hq, Hkv, d, "bf16", 1.0, 1181)[0]
    mask = torch.ones((B, 1, nblocks(Nq), nblocks(Nk)), dtype=torch.uint8)
    a = gpu_fwd_bwd(q, k, v, do, mask, 0.09, causal)
    qc, kc, vc, dc = (x.cuda() for x in (q, k, v, do))
    out_p, lse_p = attn_fwd(qc, kc, vc, 0.09, causal)
    out, lse = a[4].cuda(), a[5].cuda()
    b = [x.cpu() for x in attn_bwd(qc, kc, vc, out, dc, lse, 0.09, causal)]
    torch.cuda.synchronize()
    if causal:
        assert torch.equal(out_p.cpu(), a[4]) and torch.equal(lse_p.cpu(), a[5])
    else:
        assert (out_p.cpu().float() - a[4].float()).abs().max().item() <= 4e-3
        assert (lse_p.cpu() - a[5]).abs().max().item() <= 1e-5
    torch.cuda.synchronize()
    for x, y in zip(a[:4], b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("causal", [False, True])
def test_block_diagonal_documents_are_bitwise_per_document_attn_bwd(causal):
    # documents of whole blocks packed into one sequence, each attending to
    # itself only: the gradients equal attn_bwd run on each document alone
    from exact_tiled_attention_35_amd import attn_bwd

    docs, Hq, Hkv, d = [256, 384, 128], 4, 2, 64
    N = sum(docs)
    q, k, v = make_qkv(1, N, N, Hq, Hkv, d, "bf16", 1.0, 1182)
    do = make_qkv(1, N, N, Hq, Hkv, d, "bf16", 1.0, 1183)[0]
    mask = torch.zeros((1, 1, N // BLOCK, N // BLOCK), dtype=torch.uint8)
    s0 = 0
    for n in docs:
        mask[0, 0, s0 // BLOCK:(s0 + n) // BLOCK, s0 // BLOCK:(s0 + n) // BLOCK] = 1
        s0 += n
    dq, dk, dv, delta, outb, lseb = gpu_fwd_bwd(q, k, v, do, mask, 0.1, causal)
    s0 = 0
    for n in docs:
        sl = slice(s0, s0 + n)
        qc, kc, vc, dc = (x[:, sl].contiguous().cuda() for x in (q, k, v, do))
        # the backward of each document alone, from the same forward output
        # (a document's own attn_fwd may take the key-split kernel for its
        # small grid, whose output differs in rounding order)
        out = outb[:, sl].contiguous().cuda()
        lse = lseb[:, :, sl].contiguous().cuda()
        gq, gk, gv, gd = (x.cpu() for x in attn_bwd(qc, kc, vc, out, dc, lse, 0.1, causal))
        torch.cuda.synchronize()
        assert torch.equal(dq[:, sl], gq) and torch.equal(dk[:, sl], gk) and torch.equal(dv[:, sl], gv)
        assert torch.equal(delta[:, :, sl], gd)
        s0 += n


def test_empty_mask_gives_zero_gradients():
    q, k, v = make_qkv(1, 200, 300, 4, 2, 128, "bf16", 1.0, 1184)
    do = make_qkv(1, 200, 300, 4, 2, 128, "bf16", 1.0, 1185)[0]
    mask = torch.zeros((1, 4, 2, 3), dtype=torch.uint8)
    dq, dk, dv, _, out, lse = gpu_fwd_bwd(q, k, v, do, mask, 0.1, False)
    assert (dq == 0).all() and (dk == 0).all() and (dv == 0).all()


def test_backward_is_deterministic():
    B, Hq, Hkv, Nq, Nk, d, dt, Hm, dens = CASES[0]
    q, k, v = make_qkv(B, Nq, Nk, Hq, Hkv, d, dt, 1.0, 1186)
    do = make_qkv(B, Nq, Nk, Hq, Hkv, d, dt, 1.0, 1187)[0]
    mask = make_block_mask(B, Hm, nblocks(Nq), nblocks(Nk), dens, 1188)
    a = gpu_fwd_bwd(q, k, v, do, mask, 0.1, True)
    b = gpu_fwd_bwd(q, k, v, do, mask, 0.1, True)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_headline_workload_heads_full_size():
    """The block-sparse headline workload at full size: the gradients of two
    (batch, head) pairs (a KV group each) against the oracle."""
    name = next(iter(BLOCKSPARSE_WORKLOADS))
    spec = BLOCKSPARSE_WORKLOADS[name]
    w = WORKLOADS[spec["base"]]
    q, k, v = make_workload(w)
    do = make_qkv(w.B, w.Nq, w.Nk, w.Hq, w.Hkv, w.d, w.dtype, w.sigma, w.seed + 100)[0]
    mask = make_block_mask(w.B, w.Hq, nblocks(w.Nq), nblocks(w.Nk), spec["density"], spec["mask_seed"])
    dq, dk, dv, delta, out, lse = gpu_fwd_bwd(q, k, v, do, mask, w.scale, w.causal)
    for b, h in ((0, 0), (w.B - 1, w.Hq - 1)):
        sl = lambda x, hh=h: x[b:b + 1, :, hh:hh + 1]  # noqa: E731
        want = oracle.attention_backward(sl(q), sl(k), sl(v), sl(do), w.scale, w.causal,
                                         block_mask=mask[b:b + 1, h:h + 1])
        vis = element_mask(mask[b:b + 1, h:h + 1], 1, w.Nq, w.Nk, w.causal)
        base = lowp_backward_masked(sl(q), sl(k), sl(v), sl(do), sl(out), w.scale, vis)
        check_grads((sl(dq), sl(dk), sl(dv)), want[:3], base, f"{name} b{b} h{h}")
