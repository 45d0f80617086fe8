"""Seeded synthetic inputs for exact attention.

This module only draws random numbers and names workload shapes; it holds
none of the attention arithmetic.  It is the one module that both the GPU
path's callers (tests, bench) and the CPU oracle's callers use, so that both
sides see exactly the same input values.

Recipe: a CPU ``torch.Generator`` seeded with the workload's seed draws q, k,
v in that order as fp32 N(0, 1) samples, each multiplied by the workload's
standard deviation and rounded to nearest-even into bf16 or fp16.  The pages
measure on no dataset; their only described workloads are the README
benchmark setup (hysenlabs.com page, section "Leistungs- und Speicherangaben
im README": head dims 64/128, hidden 2048, sequence 512..16k, batch 16k/seq)
and the PyTorch example's ``torch.randn`` inputs (tokenwerk.de page, section
"Ein begrenztes SDPA-Beispiel lesen").  Layout is [B, N, H, d].
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import torch

DTYPES = {"bf16": torch.bfloat16, "fp16": torch.float16}


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    Nq: int
    Nk: int
    d: int
    dtype: str
    causal: bool
    sigma: float
    seed: int

    @property
    def scale(self) -> float:
        # 1/sqrt(d) as the fp32 value the library receives.
        return float(torch.tensor(1.0 / math.sqrt(self.d), dtype=torch.float32))

    def shapes(self):
        return ((self.B, self.Nq, self.Hq, self.d),
                (self.B, self.Nk, self.Hkv, self.d))


# The five workloads the attention-forward measurements are quoted on.
WORKLOADS = {
    w.name: w
    for w in [
        Workload("single_head_b1_h1_n1024_d64_bf16", 1, 1, 1, 1024, 1024, 64, "bf16", False, 1.0, 1),
        Workload("mha_b4_h16_n4096_d128_bf16", 4, 16, 16, 4096, 4096, 128, "bf16", False, 1.0, 2),
        Workload("causal_mha_b2_h32_n8192_d128_bf16", 2, 32, 32, 8192, 8192, 128, "bf16", True, 1.0, 3),
        Workload("causal_gqa_b1_hq64_hkv8_n16384_d128_bf16", 1, 64, 8, 16384, 16384, 128, "bf16", True, 1.0, 4),
        Workload("causal_long_b1_h16_n32768_d256_fp16", 1, 16, 16, 32768, 32768, 256, "fp16", True, 0.5, 5),
    ]
}
WORKLOAD_ORDER = list(WORKLOADS)
HEADLINE = "mha_b4_h16_n4096_d128_bf16"

# KV-cache decode: one new query row per sequence against a full cache of Nk
# rows (Nk - 1 already cached, one appended by the call), GQA 32/8, d = 128.
DECODE_WORKLOADS = {
    w.name: w
    for w in [
        Workload("decode_b16_hq32_hkv8_cache32768_d128_bf16", 16, 32, 8, 1, 32768, 128, "bf16",
                 True, 1.0, 6),
        Workload("decode_b1_hq32_hkv8_cache131072_d128_bf16", 1, 32, 8, 1, 131072, 128, "bf16",
                 True, 1.0, 7),
    ]
}


def make_qkv(B, Nq, Nk, Hq, Hkv, d, dtype="bf16", sigma=1.0, seed=0):
    """Draw q [B,Nq,Hq,d], k and v [B,Nk,Hkv,d] on the CPU, rounded to ``dtype``."""
    dt = DTYPES[dtype]
    g = torch.Generator("cpu").manual_seed(int(seed))

    def draw(shape):
        x = torch.randn(shape, generator=g, dtype=torch.float32)
        if sigma != 1.0:
            x.mul_(sigma)
        return x.to(dt)

    q = draw((B, Nq, Hq, d))
    k = draw((B, Nk, Hkv, d))
    v = draw((B, Nk, Hkv, d))
    return q, k, v


def make_workload(w: Workload):
    return make_qkv(w.B, w.Nq, w.Nk, w.Hq, w.Hkv, w.d, w.dtype, w.sigma, w.seed)


def varlen_lengths(total, lo, hi, seed):
    """Sequence lengths drawn uniformly from [lo, hi] until they sum to
    ``total`` (the last one trimmed), from a seeded CPU generator."""
    g = torch.Generator("cpu").manual_seed(int(seed))
    lens = []
    while sum(lens) < total:
        lens.append(int(torch.randint(lo, hi + 1, (1,), generator=g)))
    lens[-1] -= sum(lens) - total
    return lens


def make_varlen(lens_q, lens_k, Hq, Hkv, d, dtype="bf16", sigma=1.0, seed=0):
    """Packed q [sum(lens_q), Hq, d], k and v [sum(lens_k), Hkv, d] (CPU) and
    the int32 prefix sums cu_q, cu_k [B + 1]; values drawn as in make_qkv."""
    dt = DTYPES[dtype]
    g = torch.Generator("cpu").manual_seed(int(seed))
    tq, tk = int(sum(lens_q)), int(sum(lens_k))

    def draw(shape):
        x = torch.randn(shape, generator=g, dtype=torch.float32)
        if sigma != 1.0:
            x.mul_(sigma)
        return x.to(dt)

    q = draw((tq, Hq, d))
    k = draw((tk, Hkv, d))
    v = draw((tk, Hkv, d))
    cu_q = torch.tensor([0] + list(torch.tensor(lens_q, dtype=torch.int64).cumsum(0)), dtype=torch.int32)
    cu_k = torch.tensor([0] + list(torch.tensor(lens_k, dtype=torch.int64).cumsum(0)), dtype=torch.int32)
    return q, k, v, cu_q, cu_k


# Packed variable-length self-attention: 16384 tokens in sequences of 256 to
# 4096 tokens (the README benchmark's 16k tokens per batch and hidden 2048 as
# 16 heads of 128), seed 8; causal and not.
VARLEN_WORKLOADS = {
    n: dict(name=n, total=16384, lo=256, hi=4096, H=16, d=128, dtype="bf16", seed=8, causal=c)
    for n, c in (("varlen_causal_t16384_len256to4096_h16_d128_bf16", True),
                 ("varlen_t16384_len256to4096_h16_d128_bf16", False))
}


def make_block_mask(B, Hm, nqb, nkb, density, seed):
    """uint8 flags [B, Hm, nqb, nkb] for the block-sparse forward: each
    (query block, key block) pair is kept with probability ``density``,
    independently, from a seeded CPU generator."""
    g = torch.Generator("cpu").manual_seed(int(seed))
    return (torch.rand((B, Hm, nqb, nkb), generator=g, dtype=torch.float32) < density).to(torch.uint8)


# Block-sparse forward: the headline shape and the causal B2 H32 N8192 shape,
# each query head with its own random mask over the 128 x 128 blocks
# (density 0.5, seed 9).
BLOCK = 128
BLOCKSPARSE_WORKLOADS = {
    "blocksparse_d50_mha_b4_h16_n4096_d128_bf16":
        dict(base="mha_b4_h16_n4096_d128_bf16", density=0.5, mask_seed=9),
    "blocksparse_d50_causal_mha_b2_h32_n8192_d128_bf16":
        dict(base="causal_mha_b2_h32_n8192_d128_bf16", density=0.5, mask_seed=9),
}
