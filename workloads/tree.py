"""Seeded draft trees for tree verification.

Draft heads each propose a few high-probability candidates for one future
position, and the candidates are combined into a tree of continuations that the
target scores in one pass (the LLM inference handbook, section "Medusa").  The
synthetic drafter here: a full tree with ``branching[l]`` children per node at
depth l, numbered level by level (so every parent precedes its children), and
the children of node p are the top-k tokens of a noisy copy of the target's
logits at p (noise N(0, draft_noise_std)), most likely first.

Like ``generate``, this only draws inputs: it takes no acceptance decision and
computes no attention.
"""

from __future__ import annotations

from typing import List, Sequence, Tuple

import torch

from .generate import VerifyInputs, WorkloadSpec, _gen, generate


def tree_parents(branching: Sequence[int]) -> List[int]:
    """Parents of nodes 1..T of a full tree (level order): parents[i-1] = parent of node i."""
    parents: List[int] = []
    level = [0]
    nxt = 1
    for k in branching:
        new = []
        for p in level:
            for _ in range(int(k)):
                parents.append(p)
                new.append(nxt)
                nxt += 1
        level = new
    return parents


def tree_inputs(spec: WorkloadSpec, branching: Sequence[int], device="cpu") -> Tuple[VerifyInputs, torch.Tensor,
                                                                                   torch.Tensor]:
    """Inputs of one tree-verify step: every sequence drafts the same tree shape.

    Returns (inputs, parents int32 [T_q - B], tree_tokens int32 [T_q - B]); node i
    of sequence b sits at verify row q_start[b] + i, and its parent and token at
    index (q_start[b] - b) + i - 1.  ``spec.draft_len`` is replaced by the node
    count."""
    device = torch.device(device)
    par = tree_parents(branching)
    T = len(par)
    sp = spec.with_(draft_len=T, mode="greedy", alpha=None)
    inp = generate(sp, device=device)
    B = sp.batch
    q_start = inp.q_start.cpu()
    children: List[List[int]] = [[] for _ in range(T + 1)]
    for i, p in enumerate(par, start=1):
        children[p].append(i)
    parents = torch.tensor(par * B, dtype=torch.int32)
    tokens = torch.zeros(B * T, dtype=torch.int64, device=device)
    gen = _gen(spec.seed, "tree_noise", device)
    inner = [p for p in range(T + 1) if children[p]]
    kmax = max(len(children[p]) for p in inner) if inner else 0
    for b in range(B):
        t0 = int(q_start[b])
        rows = torch.tensor([t0 + p for p in inner], device=device)
        noisy = inp.target_logits[rows] + torch.randn((len(inner), sp.vocab), generator=gen, device=device,
                                                      dtype=torch.float32) * spec.draft_noise_std
        top = torch.topk(noisy, kmax, dim=-1).indices
        for r, p in enumerate(inner):
            for j, c in enumerate(children[p]):
                tokens[b * T + c - 1] = top[r, j]
    return inp, parents.to(device), tokens.to(torch.int32)
