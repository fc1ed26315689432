"""Seeded synthetic inputs for the speculative-decoding verify step.

This package is shared by the CPU oracle's tests, the GPU parity tests and the
benchmark. It only draws random numbers and lays them out in the buffers the
verify step consumes (paged K/V cache, block table, logits, drafted tokens,
uniforms). It computes nothing the verify step computes: no attention, no
acceptance test, no residual or inverse-CDF sampling.
"""

from .generate import VerifyInputs, WorkloadSpec, generate, draft_pool_pages
from .presets import PRESETS, preset

__all__ = ["VerifyInputs", "WorkloadSpec", "generate", "draft_pool_pages", "PRESETS", "preset"]
