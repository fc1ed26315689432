"""Seeded synthetic inputs for the speculative-decoding verify step.

This package is shared by the CPU oracle's tests, the GPU parity tests and the
benchmark. It only draws random numbers and lays them out in the buffers the
verify step consumes (paged K/V cache, block table, logits, drafted tokens,
uniforms, draft trees, and the verify rows and weight of a linear layer). It computes
nothing the verify step computes: no attention, no acceptance test, no
residual or inverse-CDF sampling, no matrix product.
"""

from .generate import VerifyInputs, WorkloadSpec, generate, draft_pool_pages
from .presets import PRESETS, preset
from .linear import EXPERT_K, EXPERT_N, linear_inputs
from .tree import tree_inputs, tree_parents

__all__ = ["VerifyInputs", "WorkloadSpec", "generate", "draft_pool_pages", "PRESETS", "preset",
           "linear_inputs", "EXPERT_N", "EXPERT_K",
           "tree_inputs", "tree_parents"]
