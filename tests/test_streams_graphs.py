"""The hot path on a caller's stream and inside a captured HIP graph (GPU).

Every entry point enqueues its kernels on the stream it is given and
allocates nothing, so a call can run on a side stream after other work on
that stream, and can be captured into a graph and replayed with new inputs
copied into the captured buffers.  Each replay is compared bit for bit with
the same call made eagerly (the kernels are deterministic)."""

import math

import pytest
import torch

from attn_workloads import make_qkv

pytestmark = pytest.mark.gpu


def test_forward_on_a_side_stream_after_pending_work():
    from exact_tiled_attention_35_amd import attn_fwd

    q, k, v = (x.cuda() for x in make_qkv(2, 700, 900, 8, 2, 128, "bf16", 1.0, 1300))
    ref, rl = attn_fwd(q, k, v, None, True)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        torch.cuda._sleep(20_000_000)  # keep the stream busy before q is written
        q2 = q * 1  # written on s, after the sleep
        out, lse = attn_fwd(q2, k, v, None, True)  # must run on s, after q2
    s.synchronize()
    assert torch.equal(out, ref) and torch.equal(lse, rl)


def test_forward_and_backward_replayed_from_a_graph():
    from exact_tiled_attention_35_amd import attn_bwd, attn_fwd

    shape = (2, 300, 500, 4, 2, 64, "fp16")
    q, k, v = (x.cuda() for x in make_qkv(*shape, 1.0, 1301))
    do = make_qkv(2, 300, 300, 4, 4, 64, "fp16", 1.0, 1302)[0].cuda()
    scale = 1.0 / math.sqrt(64)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm-up outside the capture
        out, lse = attn_fwd(q, k, v, scale, True)
        attn_bwd(q, k, v, out, do, lse, scale, True)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        g_out, g_lse = attn_fwd(q, k, v, scale, True)
        g_dq, g_dk, g_dv, g_delta = attn_bwd(q, k, v, g_out, do, g_lse, scale, True)
    for rep in range(3):
        nq, nk, nv = (x.cuda() for x in make_qkv(*shape, 1.0, 1310 + rep))
        q.copy_(nq)
        k.copy_(nk)
        v.copy_(nv)
        g.replay()
        torch.cuda.synchronize()
        e_out, e_lse = attn_fwd(q, k, v, scale, True)
        e_dq, e_dk, e_dv, e_delta = attn_bwd(q, k, v, e_out, do, e_lse, scale, True)
        torch.cuda.synchronize()
        assert torch.equal(g_out, e_out) and torch.equal(g_lse, e_lse), rep
        assert torch.equal(g_dq, e_dq) and torch.equal(g_dk, e_dk) and torch.equal(g_dv, e_dv), rep
        assert torch.equal(g_delta, e_delta), rep


def test_decode_steps_replayed_from_a_graph():
    # A serving loop: one captured decode step (append one row, attend),
    # replayed with new query/key/value rows while cache_seqlens advances.
    from exact_tiled_attention_35_amd import attn_decode

    B, Hq, Hkv, d, Ncap = 3, 8, 2, 128, 600
    _, kc, vc = make_qkv(B, 1, Ncap, 1, Hkv, d, "bf16", 1.0, 1320)
    kc_g, vc_g = kc.cuda(), vc.cuda()
    kc_e, vc_e = kc_g.clone(), vc_g.clone()
    sl_g = torch.tensor([10, 257, 400], dtype=torch.int32, device="cuda")
    sl_e = sl_g.clone()
    q = torch.zeros(B, 1, Hq, d, dtype=torch.bfloat16, device="cuda")
    kn = torch.zeros(B, 1, Hkv, d, dtype=torch.bfloat16, device="cuda")
    vn = torch.zeros_like(kn)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm-up outside the capture (writes row sl of the copies)
        attn_decode(q, kc_g.clone(), vc_g.clone(), sl_g, kn, vn)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        g_out, g_lse = attn_decode(q, kc_g, vc_g, sl_g, kn, vn, num_splits=3)
    for step in range(4):
        nq = make_qkv(B, 1, 1, Hq, Hq, d, "bf16", 1.0, 1330 + step)[0].cuda()
        _, nk, nv = make_qkv(B, 1, 1, 1, Hkv, d, "bf16", 1.0, 1340 + step)
        q.copy_(nq)
        kn.copy_(nk.cuda())
        vn.copy_(nv.cuda())
        g.replay()
        e_out, e_lse = attn_decode(q, kc_e, vc_e, sl_e, kn, vn, num_splits=3)
        torch.cuda.synchronize()
        assert torch.equal(g_out, e_out) and torch.equal(g_lse, e_lse), step
        sl_g += 1
        sl_e += 1
    torch.cuda.synchronize()
    assert torch.equal(kc_g, kc_e) and torch.equal(vc_g, vc_e)
