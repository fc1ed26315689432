"""Relaxed (lossy) acceptance, fp64 reference — test infrastructure only.

Adaptive speculative decoding may relax how strictly the target checks each
draft token: tokens that are close enough pass, generation speeds up, and the
output leaves the target's exact distribution (the LLM inference handbook,
section on what adaptive speculative decoding can adapt: the acceptance
criterion).  AdaSD (same handbook, section "AdaSD") works from two runtime
statistics of the two models' token distributions over one shared vocabulary:
the entropy of the draft distribution, which tells the drafter when to stop
proposing, and the Jensen-Shannon distance between the draft and the target
distributions, which decides whether a draft token is close enough to the
target distribution to be accepted.

Readings (the pages name the statistics and their roles, not the formulas nor
how the threshold enters the test):
  * H(q_i) = -sum_j q_i(j) ln q_i(j), in nats, q_i = softmax of draft row i;
  * JS(p_i, q_i) = sqrt(JSD) with JSD = KL(p||m)/2 + KL(q||m)/2, m = (p+q)/2,
    natural logarithms (so 0 <= JS <= sqrt(ln 2)), p_i = softmax of target
    row i;
  * draft x_{i+1} passes when the lossless test passes (greedy: x is the
    target's top token at row i; stochastic: u_i < p(x)/q(x), as in
    oracle.accept) or when JS(p_i, q_i) <= tau; a token outside [0, V) never
    passes; what follows the first failure is the lossless rule's (greedy: the
    target's top token at row n; stochastic: a sample of max(0, p - q) at row
    n, or of p at row D when every draft passed);
  * tau < 0 switches the relaxation off: the result is the lossless one;
  * both statistics are reported for every drafted row, also past the first
    failure.
"""

from __future__ import annotations

import math
from typing import List, Optional, Tuple

import numpy as np

from .accept import _inverse_cdf, _seq_bounds, row_log_normalizer


def _probs(row) -> np.ndarray:
    r = np.asarray(row, dtype=np.float64)
    return np.exp(r - row_log_normalizer(r))


def row_entropy(logits_row) -> float:
    """Entropy in nats of softmax(logits_row), with 0 ln 0 = 0."""
    p = _probs(logits_row)
    nz = p > 0
    return float(-(p[nz] * np.log(p[nz])).sum())


def js_distance(target_row, draft_row) -> float:
    """Jensen-Shannon distance (natural log) between softmax(target_row) and
    softmax(draft_row): the square root of the mean of KL(p||m) and KL(q||m),
    m = (p+q)/2."""
    p, q = _probs(target_row), _probs(draft_row)
    m = 0.5 * (p + q)
    kp = float((p[p > 0] * np.log(p[p > 0] / m[p > 0])).sum())
    kq = float((q[q > 0] * np.log(q[q > 0] / m[q > 0])).sum())
    return math.sqrt(max(0.0, 0.5 * (kp + kq)))


def accept_lossy(mode: str, target_logits, draft_logits, draft_tokens, q_start, uniforms, js_threshold: float,
                 margins: Optional[dict] = None) -> Tuple[np.ndarray, np.ndarray, np.ndarray, np.ndarray]:
    """Acceptance relaxed by the JS distance.  Returns (accept_len [B],
    out_tokens [T_q], draft_entropy [T_q - B], js_distance [T_q - B]).

    If ``margins`` is a dict it receives "test" (|u - r| / r of stochastic
    tests, as oracle.accept), "js" (|JS - tau| wherever the JS test decided a
    position) and "sample" (relative distance of u*Z to the nearest CDF step)."""
    if mode not in ("greedy", "stochastic"):
        raise ValueError(mode)
    target = np.asarray(target_logits, dtype=np.float32)
    draft = np.asarray(draft_logits, dtype=np.float32)
    tokens = np.asarray(draft_tokens)
    q_start = np.asarray(q_start)
    u_all = np.asarray(uniforms, dtype=np.float32) if uniforms is not None else None
    B = len(q_start) - 1
    T, V = target.shape
    tau = float(js_threshold)
    al = np.zeros(B, dtype=np.int32)
    out = np.full(T, -1, dtype=np.int32)
    ent = np.zeros(T - B, dtype=np.float64)
    jsd = np.zeros(T - B, dtype=np.float64)
    test_m: List[float] = []
    js_m: List[float] = []
    samp_m: List[float] = []
    with np.errstate(invalid="ignore", over="ignore", divide="ignore"):
        for b in range(B):
            t0, D, d0 = _seq_bounds(q_start, b)
            for i in range(D):
                ent[d0 + i] = row_entropy(draft[d0 + i])
                jsd[d0 + i] = js_distance(target[t0 + i], draft[d0 + i])
            n = 0
            while n < D:
                x = int(tokens[d0 + n])
                if not (0 <= x < V):
                    break
                if mode == "greedy":
                    strict = x == int(np.argmax(target[t0 + n]))
                else:
                    lp = float(target[t0 + n, x]) - row_log_normalizer(target[t0 + n])
                    lq = float(draft[d0 + n, x]) - row_log_normalizer(draft[d0 + n])
                    r = float(np.exp(np.float64(lp - lq)))
                    u = float(u_all[t0 + n])
                    if r > 0 and math.isfinite(r):
                        test_m.append(abs(u - r) / r)
                    strict = u < r
                if not strict:
                    if tau >= 0:
                        js_m.append(abs(jsd[d0 + n] - tau))
                    if not (jsd[d0 + n] <= tau):
                        break
                out[t0 + n] = x
                n += 1
            if mode == "greedy":
                out[t0 + n] = int(np.argmax(target[t0 + n]))
            else:
                p = _probs(target[t0 + n])
                w = np.maximum(0.0, p - _probs(draft[d0 + n])) if n < D else p
                if not (w.sum() > 0):
                    w = p
                y, m = _inverse_cdf(w, float(u_all[t0 + D]))
                samp_m.append(m)
                out[t0 + n] = y
            al[b] = n + 1
    if margins is not None:
        margins["test"] = np.asarray(test_m)
        margins["js"] = np.asarray(js_m)
        margins["sample"] = np.asarray(samp_m)
    return al, out, ent, jsd
