"""Verify-shaped linear layer, fp64 reference — test infrastructure only.

With speculation, every linear layer of the target model sees M*(1+D) rows in
the verify pass instead of M: the GEMM-M grows by the factor 1+D while the
weight stays the same ("Co-Designing AI Models Using Speculative Decoding for
Faster LLM Inference", translated page, section "Draft length and performance
of linear layers", with its Figure 3 for a representative expert GEMM of
N = K = 6144).  The layer computes, for the verify rows x of shape [M', K]
(M' = M*(1+D)) and the weight W of shape [N, K] (one row per output feature):

    y[m, n] = sum_k x[m, k] * W[n, k]

This module is that definition, with the bf16 inputs widened exactly to fp64
and the sums taken in fp64 (numpy's matmul of the widened operands).
``linear_abs_sum`` gives sum_k |x[m, k] * W[n, k]|, the scale of the rounding
error a lower-precision accumulation of the same sum can make.
"""

from __future__ import annotations

import numpy as np

from .attention import bf16_bits_to_f64


def _widen(bits) -> np.ndarray:
    a = np.asarray(bits)
    if a.dtype in (np.uint16, np.int16):
        return bf16_bits_to_f64(a)
    return a.astype(np.float64)


def verify_linear(x, w) -> np.ndarray:
    """y = x W^T in fp64.  x: [M, K] and w: [N, K], as bf16 bit patterns
    (uint16/int16) or real arrays; returns fp64 [M, N]."""
    xf, wf = _widen(x), _widen(w)
    if xf.ndim != 2 or wf.ndim != 2 or xf.shape[1] != wf.shape[1]:
        raise ValueError(f"x {xf.shape} and w {wf.shape} must be [M, K] and [N, K]")
    return xf @ wf.T


def linear_abs_sum(x, w) -> np.ndarray:
    """sum_k |x[m, k] W[n, k]| in fp64, [M, N]."""
    return np.abs(_widen(x)) @ np.abs(_widen(w)).T
