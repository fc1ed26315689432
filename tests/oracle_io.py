"""Marshalling of generated torch tensors into the numpy arrays the oracle takes."""

import numpy as np
import torch


def bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> its uint16 bit patterns on the host."""
    assert t.dtype == torch.bfloat16
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def host(t):
    return None if t is None else t.detach().cpu().numpy()


def v_layout(inp) -> str:
    """'key' when the V pages are stored like K ([P, H, page, d]), else 'dim'
    ([P, H, d, page]); head_dim is never the page size here."""
    return "key" if tuple(inp.v_cache.shape) == tuple(inp.k_cache.shape) else "dim"


def attention_args(inp):
    return dict(q_bits=bits(inp.q), k_bits=bits(inp.k_cache), v_bits=bits(inp.v_cache),
                block_table=host(inp.block_table), kv_len=host(inp.kv_len),
                q_start=host(inp.q_start), group=inp.group, v_layout=v_layout(inp))


def accept_args(inp):
    return dict(target_logits=host(inp.target_logits), draft_logits=host(inp.draft_logits),
                draft_tokens=host(inp.draft_tokens), q_start=host(inp.q_start),
                uniforms=host(inp.uniforms))
