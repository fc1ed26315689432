"""The speculative-decoding verify step on AMD Instinct MI355X (gfx950).

Verify attention over a paged bf16 KV cache and vocab-parallel accept/reject
(plus draft-tree verification, acceptance relaxed by the Jensen-Shannon
distance, a closed adaptive-speculation loop on a toy LM, and the
verify-shaped linear layer y = x W^T), as hand-written HIP
kernels behind a C ABI (``include/sd_verify.h``,
``libsdverify.so``).  This package is the Python binding of that ABI: it
marshals PyTorch device tensors and the current stream into the C calls.
"""

import torch  # noqa: F401  (load torch's HIP runtime before libsdverify.so)

from .binding import (  # noqa: F401
    SdError,
    accept_desc,
    attn_desc,
    lib,
    linear_desc,
    loop_desc,
    sd_accept_lossy,
    sd_accept_lossy_workspace_size,
    sd_accept_reject,
    sd_accept_reject_noalloc,
    sd_accept_reject_workspace_size,
    sd_closed_loop,
    sd_closed_loop_workspace_size,
    sd_last_error,
    sd_verify_attention,
    sd_verify_attention_workspace_size,
    sd_verify_linear,
    sd_verify_linear_workspace_size,
    sd_verify_step,
    sd_verify_step_workspace_size,
    sd_verify_tree_attention,
    sd_tree_accept,
    sd_tree_accept_workspace_size,
    sd_version,
    sd_validate_inputs,
    SD_BAD,
)

__all__ = [
    "SdError", "accept_desc", "attn_desc", "lib", "sd_accept_reject", "sd_accept_reject_workspace_size",
    "sd_last_error", "sd_verify_attention", "sd_verify_attention_workspace_size", "sd_verify_step",
    "sd_verify_step_workspace_size", "sd_version", "linear_desc", "sd_verify_linear",
    "sd_verify_linear_workspace_size", "sd_verify_tree_attention", "sd_tree_accept", "sd_tree_accept_workspace_size",
    "sd_accept_lossy", "sd_accept_lossy_workspace_size", "loop_desc", "sd_closed_loop", "sd_closed_loop_workspace_size",
    "sd_validate_inputs", "SD_BAD", "sd_accept_reject_noalloc",
]
