"""Seeded inputs for the verify-shaped linear layer.

x  bf16 [M, K]  the verify rows (M = batch * (1+D)), N(0, 1)
w  bf16 [N, K]  one row per output feature, N(0, 1/K), so outputs are O(1)

Both are drawn in fp32 from their own seeded generators and rounded to bf16
(nearest even).  M, N and K default to the expert GEMM of the translated
co-design page (N = K = 6144).
"""

from __future__ import annotations

import math

import torch

from .generate import _gen

EXPERT_N = 6144
EXPERT_K = 6144


def linear_inputs(m: int, n: int = EXPERT_N, k: int = EXPERT_K, seed: int = 0, device="cpu"):
    dev = torch.device(device)
    x = torch.randn(m, k, generator=_gen(seed, "linear_x", dev), device=dev, dtype=torch.float32)
    w = torch.randn(n, k, generator=_gen(seed, "linear_w", dev), device=dev, dtype=torch.float32)
    return x.to(torch.bfloat16), (w / math.sqrt(k)).to(torch.bfloat16)
