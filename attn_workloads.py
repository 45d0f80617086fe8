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
