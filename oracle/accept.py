"""Accept / reject over the vocabulary, fp64 reference — test infrastructure only.

Per sequence b the verify step has 1+D_b target rows t_0..t_D (row i is the
target's next-token distribution after position i), D_b draft rows
d_0..d_{D-1} (the distribution draft x_{i+1} was drawn from) and the drafts
x_1..x_D.  Acceptance walks the drafts left to right, stops at the first
failure, and always adds one token from the target, so the acceptance length
AL lies in [1, 1+D] (NVIDIA co-design page, "What is speculative decoding?";
LLM inference handbook, "How speculative decoding works", steps 3-4).

Greedy: draft x_{i+1} passes when it equals the target's top token at row i
(the co-design page: the target accepts proposals until the first mismatch).
The emitted tokens are x_1..x_n followed by the target's top token at row n.
The top token is taken on the fp32 logits, lowest token id on ties.

Stochastic ("How does speculative decoding speed up LLM inference?",
"Mechanism" and "Math intuition"): with p = softmax(t_i), q = softmax(d_i),
draft x passes with probability min(1, p(x)/q(x)).  Here that is the test
u_i < r_i with r_i = exp(log p(x) - log q(x)) computed from the fp32 logits in
fp64; u_i is the caller's uniform.  At the first failure, row n, the token is
resampled from the residual max(0, p - q) renormalised; when every draft
passes, the extra token is sampled from p at row D.  Sampling is the inverse
CDF over ascending token ids: with C_j the inclusive prefix sums of the
weights w and Z = C_{V-1}, the token is the smallest j with C_j > u * Z.

Readings where the pages are silent (all fixed here, the kernel follows them):
  * uniforms: u[q_start[b]+i] tests draft i+1; u[q_start[b]+D_b] samples;
    uniforms of tests after the first failure are skipped, not shifted;
  * q(x) = 0 < p(x) gives r = inf (pass); p(x) = 0 gives r = 0 or NaN (fail);
    a draft token outside [0, V) fails;
  * a residual that sums to zero (possible only through rounding) falls back
    to p at that row; a u*Z at or past the last prefix sum (rounding) takes
    the last token with positive weight;
  * temperature 1, no top-k / top-p.
"""

from __future__ import annotations

import math
from typing import List, Optional, Tuple

import numpy as np


def row_log_normalizer(row) -> float:
    """log sum_j exp(row_j) in fp64 (the log-partition of one logit row)."""
    r = np.asarray(row, dtype=np.float64)
    m = r.max()
    return float(m + math.log(np.exp(r - m).sum()))


def _seq_bounds(q_start, b):
    t0 = int(q_start[b])
    D = int(q_start[b + 1]) - t0 - 1
    if D < 0:
        raise ValueError("every sequence has at least one verify row")
    return t0, D, t0 - b


def accept_greedy(target_logits, draft_tokens, q_start) -> Tuple[np.ndarray, np.ndarray]:
    """Greedy first-mismatch acceptance.  Returns (accept_len [B], out_tokens [T_q])."""
    target = np.asarray(target_logits, dtype=np.float32)
    tokens = np.asarray(draft_tokens)
    q_start = np.asarray(q_start)
    B = len(q_start) - 1
    T = target.shape[0]
    al = np.zeros(B, dtype=np.int32)
    out = np.full(T, -1, dtype=np.int32)
    for b in range(B):
        t0, D, d0 = _seq_bounds(q_start, b)
        n = 0
        while n < D:
            top = int(np.argmax(target[t0 + n]))       # first maximum = lowest id
            if int(tokens[d0 + n]) != top:
                break
            out[t0 + n] = int(tokens[d0 + n])
            n += 1
        out[t0 + n] = int(np.argmax(target[t0 + n]))
        al[b] = n + 1
    return al, out


def _inverse_cdf(w: np.ndarray, u: float) -> Tuple[int, float]:
    """Smallest j with C_j > u*Z (C = inclusive prefix sums, ascending j).

    Returns (token, margin) where margin is the distance of u*Z to the nearest
    prefix sum, relative to Z.
    """
    C = np.cumsum(w)
    Z = C[-1]
    T = float(u) * Z
    j = int(np.searchsorted(C, T, side="right"))
    if j >= len(w):
        j = int(np.nonzero(w > 0)[0][-1])
    margin = float(np.min(np.abs(C - T)) / Z)
    return j, margin


def accept_stochastic(target_logits, draft_logits, draft_tokens, q_start, uniforms,
                      margins: Optional[dict] = None) -> Tuple[np.ndarray, np.ndarray]:
    """min(1, p/q) acceptance with residual resampling and the extra token.

    Returns (accept_len [B], out_tokens [T_q]).  If ``margins`` is a dict it
    receives "test" (|u - r| / r per executed test) and "sample" (relative
    distance of u*Z to the nearest CDF step per sequence).
    """
    target = np.asarray(target_logits, dtype=np.float32)
    draft = np.asarray(draft_logits, dtype=np.float32)
    tokens = np.asarray(draft_tokens)
    u_all = np.asarray(uniforms, dtype=np.float32)
    q_start = np.asarray(q_start)
    B = len(q_start) - 1
    T, V = target.shape
    al = np.zeros(B, dtype=np.int32)
    out = np.full(T, -1, dtype=np.int32)
    test_m: List[float] = []
    samp_m: List[float] = []
    with np.errstate(invalid="ignore", over="ignore", divide="ignore"):
        for b in range(B):
            t0, D, d0 = _seq_bounds(q_start, b)
            n = 0
            while n < D:
                x = int(tokens[d0 + n])
                if not (0 <= x < V):
                    break
                lp = float(target[t0 + n, x]) - row_log_normalizer(target[t0 + n])
                lq = float(draft[d0 + n, x]) - row_log_normalizer(draft[d0 + n])
                r = float(np.exp(np.float64(lp - lq)))      # inf when q(x) = 0, nan when both 0
                u = float(u_all[t0 + n])
                if r > 0 and math.isfinite(r):
                    test_m.append(abs(u - r) / r)
                if not (u < r):
                    break
                out[t0 + n] = x
                n += 1
            t_row = target[t0 + n].astype(np.float64)
            p = np.exp(t_row - row_log_normalizer(t_row))
            if n < D:
                d_row = draft[d0 + n].astype(np.float64)
                q = np.exp(d_row - row_log_normalizer(d_row))
                w = np.maximum(0.0, p - q)
            else:
                w = p
            if not (w.sum() > 0):
                w = p
            y, m = _inverse_cdf(w, float(u_all[t0 + D]))
            samp_m.append(m)
            out[t0 + n] = y
            al[b] = n + 1
    if margins is not None:
        margins["test"] = np.asarray(test_m)
        margins["sample"] = np.asarray(samp_m)
    return al, out


def accept_reject(mode: str, target_logits, draft_logits, draft_tokens, q_start, uniforms=None,
                  margins: Optional[dict] = None):
    if mode == "greedy":
        return accept_greedy(target_logits, draft_tokens, q_start)
    if mode == "stochastic":
        return accept_stochastic(target_logits, draft_logits, draft_tokens, q_start, uniforms, margins)
    raise ValueError(mode)
