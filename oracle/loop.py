"""Closed speculative-decoding loop on a toy LM, plain reference — test
infrastructure only.

The loop (the LLM inference handbook, section on SGLang's adaptive
speculative decoding): every round drafts D tokens per sequence, verifies them
in one pass, accepts a prefix, then measures the accepted length; an
exponential moving average (EMA) of the acceptance length picks the round
after's D among a few tiers (default [1, 3, 7]), each tier with its own
captured graph.  Only the speculation length changes, so the loop is lossless:
its output is plain greedy decoding of the target.

Pieces, all plain:
  * target: a bigram toy LM, logits of the next token = W[previous token]
    (W fp32 [V, V]); greedy acceptance as oracle.accept.accept_greedy;
  * drafter, model-free n-gram (prompt lookup): the latest earlier occurrence
    of the history's last k tokens (k = n, then n-1, ..., 1) proposes the D
    tokens that followed it; slots it cannot fill are -1 (never accepted);
  * controller (reading; the section gives no formula): ema <- (1-w) ema + w
    mean(AL) over the sequences that appended, starting from ema = 1; the next
    D is the smallest tier >= ema, else the largest tier;
  * a sequence appends its AL emitted tokens; one that would pass max_len
    appends nothing and reports AL 0 from then on.
"""

from __future__ import annotations

from typing import List, Sequence, Tuple

import numpy as np

from .accept import accept_greedy


def greedy_decode(W, history: Sequence[int], n_new: int) -> List[int]:
    """The target's plain greedy continuation: n_new tokens after `history`."""
    W = np.asarray(W, dtype=np.float32)
    out = []
    last = int(history[-1])
    for _ in range(n_new):
        last = int(np.argmax(W[last]))          # first maximum = lowest id
        out.append(last)
    return out


def ngram_draft(history: Sequence[int], n: int, D: int) -> List[int]:
    """D proposed tokens after `history` (-1 where there are none)."""
    h = [int(t) for t in history]
    L = len(h)
    for k in range(min(n, L - 1), 0, -1):
        suffix = h[L - k:]
        for j in range(L - k - 1, -1, -1):       # latest occurrence first, ending before the suffix
            if h[j:j + k] == suffix:
                nxt = h[j + k:j + k + D]
                return nxt + [-1] * (D - len(nxt))
    return [-1] * D


def next_tier(ema: float, tiers: Sequence[int]) -> int:
    for d in sorted(tiers):
        if d >= ema:
            return d
    return max(tiers)


def closed_loop(W, histories: Sequence[Sequence[int]], tiers: Sequence[int], ngram: int, ema_weight: float,
                steps: int, max_len: int) -> Tuple[List[List[int]], np.ndarray, np.ndarray]:
    """Run `steps` rounds.  Returns (histories, AL trace [steps, B], D trace [steps])."""
    W = np.asarray(W, dtype=np.float32)
    hs = [[int(t) for t in h] for h in histories]
    B = len(hs)
    al_trace = np.zeros((steps, B), dtype=np.int32)
    d_trace = np.zeros(steps, dtype=np.int32)
    ema = 1.0
    D = next_tier(ema, tiers)
    for s in range(steps):
        d_trace[s] = D
        drafts = [ngram_draft(h, ngram, D) for h in hs]
        # verify rows: the last token, then the drafts; target row i = W[row token i]
        rows = []
        for h, dr in zip(hs, drafts):
            rows.append(h[-1])
            rows.extend(dr)
        target = W[np.clip(np.asarray(rows), 0, W.shape[0] - 1)]
        tokens = np.asarray([t for dr in drafts for t in dr], dtype=np.int64)
        q_start = np.arange(B + 1) * (1 + D)
        al, out = accept_greedy(target, tokens, q_start)
        appended = []
        for b in range(B):
            a = int(al[b])
            if len(hs[b]) + a > max_len:
                a = 0
            hs[b].extend(int(t) for t in out[b * (1 + D):b * (1 + D) + a])
            al_trace[s, b] = a
            if a > 0:
                appended.append(a)
        if appended:
            ema = (1.0 - ema_weight) * ema + ema_weight * float(np.mean(appended))
        D = next_tier(ema, tiers)
    return hs, al_trace, d_trace
