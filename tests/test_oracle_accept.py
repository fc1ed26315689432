"""Pins of the accept/reject oracle against what the pages and the mathematics fix.

* Greedy speculation emits exactly the stream of plain greedy decoding (the
  NVIDIA co-design page, "What is speculative decoding?": only tokens the
  target accepts are kept, so the output equals standard decoding) — brute
  force on a seeded toy Markov language model.
* Sampling reproduces p exactly ("How does speculative decoding speed up LLM
  inference?", "Math intuition"): exact integration over the uniforms on
  midpoint grids for tiny vocabularies, chi-square over seeded trials at the
  tiny workload's sizes, and the joint law of three tokens under a toy Markov
  model.
* Mean acceptance length under a fixed acceptance rate alpha equals
  tau = (1 - alpha^(gamma+1)) / (1 - alpha) (LLM inference handbook, "Key
  metrics"), and the AL histogram is the truncated geometric law.
* AL lies in [1, 1+D]; p == q accepts everything; D = 0 is plain sampling.
"""

import math

import numpy as np
import pytest
import torch
from scipy import stats

from oracle import accept_greedy, accept_stochastic
from workloads import generate, preset
from tests.oracle_io import accept_args


def _softmax(x):
    x = np.asarray(x, dtype=np.float64)
    e = np.exp(x - x.max(-1, keepdims=True))
    return e / e.sum(-1, keepdims=True)


# ----------------------------------------------------------------------------- greedy

class ToyLM:
    """Order-2 Markov 'language model' given by a seeded logit table."""

    def __init__(self, V, seed, std=2.0):
        rng = np.random.default_rng(seed)
        self.V = V
        self.table = (rng.standard_normal((V, V, V)) * std).astype(np.float32)

    def logits(self, ctx):
        return self.table[ctx[-2], ctx[-1]]


def _plain_greedy(lm, prompt, n):
    s = list(prompt)
    while len(s) < len(prompt) + n:
        s.append(int(np.argmax(lm.logits(s))))
    return s[len(prompt):]


def _speculative_greedy(target, drafter, prompt, n, D):
    s = list(prompt)
    while len(s) < len(prompt) + n:
        ctx = list(s)
        drafts = []
        for _ in range(D):
            x = int(np.argmax(drafter.logits(ctx)))
            drafts.append(x)
            ctx.append(x)
        rows = np.stack([target.logits(s + drafts[:i]) for i in range(D + 1)])
        al, out = accept_greedy(rows, np.asarray(drafts, np.int32), np.asarray([0, D + 1], np.int32))
        assert 1 <= al[0] <= D + 1
        assert np.all(out[al[0]:] == -1)
        s.extend(int(t) for t in out[: al[0]])
    return s[len(prompt):len(prompt) + n]


@pytest.mark.parametrize("D", [1, 3, 6])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_greedy_speculation_equals_plain_greedy_decoding(D, seed):
    V = 12
    target = ToyLM(V, seed)
    drafter = ToyLM(V, seed)
    rng = np.random.default_rng(100 + seed)
    drafter.table = drafter.table + rng.standard_normal(drafter.table.shape).astype(np.float32) * 1.5
    prompt = [int(rng.integers(V)), int(rng.integers(V))]
    assert _speculative_greedy(target, drafter, prompt, 64, D) == _plain_greedy(target, prompt, 64)


def test_greedy_edges():
    rng = np.random.default_rng(0)
    rows = rng.standard_normal((4, 50)).astype(np.float32)
    top = rows.argmax(1).astype(np.int32)
    qs = np.asarray([0, 4], np.int32)
    al, out = accept_greedy(rows, top[:3], qs)            # drafts == target's choice
    assert al[0] == 4 and list(out) == list(top)
    bad = top[:3].copy()
    bad[0] = (bad[0] + 1) % 50                            # first draft wrong
    al, out = accept_greedy(rows, bad, qs)
    assert al[0] == 1 and out[0] == top[0] and np.all(out[1:] == -1)
    # ties: the lowest token id is the target's choice
    rows2 = np.zeros((1, 7), np.float32)
    rows2[0, [2, 5]] = 3.0
    al, out = accept_greedy(rows2, np.zeros(0, np.int32), np.asarray([0, 1], np.int32))
    assert al[0] == 1 and out[0] == 2
    # out-of-range draft ids fail
    al, out = accept_greedy(rows, np.asarray([-1, 7, 7], np.int32), qs)
    assert al[0] == 1


# ----------------------------------------------------------------------------- exactness

def _grid(M):
    return ((np.arange(M) + 0.5) / M).astype(np.float32)


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_first_token_law_is_p_by_integration_over_uniforms(seed):
    """P(first token = y) = sum_x q(x) [A(x) 1{y=x} + (1-A(x)) R(x,y)] = p(y),
    where A and R are measured on the oracle itself over midpoint grids of u."""
    rng = np.random.default_rng(seed)
    V, M = 5, 4096
    t = (rng.standard_normal(V) * 1.5).astype(np.float32)
    d = (t + rng.standard_normal(V) * 1.0).astype(np.float32)
    d[rng.integers(V)] = -np.inf if seed == 3 else d[0]   # a zero of q in one case
    p, q = _softmax(t), _softmax(d)
    u = _grid(M)
    law = np.zeros(V)
    for x in range(V):
        if q[x] == 0:
            continue
        B = M
        tgt = np.tile(np.stack([t, t]), (B, 1))          # rows: target row 0, target row 1
        drf = np.tile(d[None], (B, 1))
        qs = (np.arange(B + 1) * 2).astype(np.int32)
        toks = np.full(B, x, np.int32)
        # A(x): vary the test uniform, fixed sample uniform
        uni = np.stack([u, np.full(B, 0.5, np.float32)], 1).reshape(-1)
        al, out = accept_stochastic(tgt, drf, toks, qs, uni)
        A = np.mean(al == 2)
        assert abs(A - min(1.0, p[x] / q[x])) <= 1.0 / M
        # R(x, .): force the rejection (u just below 1), vary the sample uniform
        uni = np.stack([np.full(B, np.float32(1 - 2**-24)), u], 1).reshape(-1)
        al, out = accept_stochastic(tgt, drf, toks, qs, uni)
        rej = al == 1
        R = np.bincount(out[0::2][rej], minlength=V) / M if rej.any() else np.zeros(V)
        if rej.any():
            resid = np.maximum(p - q, 0)
            np.testing.assert_allclose(R, resid / resid.sum(), atol=1.0 / M)
        law += q[x] * (A * (np.arange(V) == x) + (1 - A) * R)
    np.testing.assert_allclose(law, p, atol=3.0 / M)


def test_d0_is_inverse_cdf_sampling_of_p():
    rng = np.random.default_rng(7)
    V, M = 9, 8192
    t = (rng.standard_normal(V) * 2).astype(np.float32)
    t[4] = -np.inf                                      # a zero-probability token is never drawn
    p = _softmax(t)
    u = _grid(M)
    al, out = accept_stochastic(np.tile(t, (M, 1)), np.zeros((0, V), np.float32), np.zeros(0, np.int32),
                                np.arange(M + 1, dtype=np.int32), u)
    assert np.all(al == 1)
    freq = np.bincount(out, minlength=V) / M
    np.testing.assert_allclose(freq, p, atol=1.0 / M)
    assert freq[4] == 0
    # monotone in u: the inverse CDF walks token ids upward
    assert np.all(np.diff(out) >= 0)


def test_tiny_workload_emitted_tokens_follow_p_chi_square():
    """At the tiny workload's sizes (V=1000, D=3, N(0,2) target, +N(0,0.5) draft):
    the token emitted at index k, given AL > k, is distributed as p_k."""
    spec = preset("tiny")
    base = generate(spec.with_(batch=1, seed=0))
    t = base.target_logits.numpy()                     # [4, V]
    d = base.draft_logits.numpy()                      # [3, V]
    V, D = t.shape[1], 3
    n_trials = 6000
    rng = np.random.default_rng(42)
    qd = _softmax(d)
    toks = np.stack([rng.choice(V, size=n_trials, p=qd[i]) for i in range(D)], 1).astype(np.int32).reshape(-1)
    uni = rng.random((n_trials, D + 1), dtype=np.float32).reshape(-1)
    al, out = accept_stochastic(np.tile(t, (n_trials, 1)), np.tile(d, (n_trials, 1)), toks,
                                np.arange(n_trials + 1, dtype=np.int32) * (D + 1), uni)
    assert al.min() >= 1 and al.max() <= D + 1
    out = out.reshape(n_trials, D + 1)
    p = _softmax(t)
    for k in range(D + 1):
        sel = al > k
        if sel.sum() < 400:
            continue
        y = out[sel, k]
        order = np.argsort(-p[k])
        cum = np.cumsum(p[k][order])
        bins = np.minimum((cum * 20).astype(int), 19)  # 20 bins of (about) equal p-mass
        bin_of = np.empty(V, int)
        bin_of[order] = bins
        obs = np.bincount(bin_of[y], minlength=20)
        exp = np.bincount(bin_of, weights=p[k], minlength=20) * sel.sum()
        keep = exp > 0
        chi = stats.chisquare(obs[keep], exp[keep] * obs[keep].sum() / exp[keep].sum())
        assert chi.pvalue > 1e-4, (k, chi)


def test_three_token_joint_law_under_toy_markov_model():
    """Repeated draft/verify cycles on an order-1 Markov model (V=4, D=2):
    the first three emitted tokens follow the target's joint law."""
    V, D, N = 4, 2, 30000
    rng = np.random.default_rng(5)
    T = (rng.standard_normal((V, V)) * 1.0).astype(np.float32)    # target logits given last token
    Q = (T + rng.standard_normal((V, V)) * 1.2).astype(np.float32)
    pT, pQ = _softmax(T), _softmax(Q)
    seqs = [[0] for _ in range(N)]
    while True:
        todo = [i for i in range(N) if len(seqs[i]) < 4]
        if not todo:
            break
        tgt, drf, toks = [], [], []
        for i in todo:
            ctx = seqs[i][-1]
            xs = []
            for _ in range(D):
                x = int(rng.choice(V, p=pQ[ctx]))
                drf.append(Q[ctx])
                xs.append(x)
                ctx = x
            chain = [seqs[i][-1]] + xs
            tgt.extend(T[c] for c in chain)
            toks.extend(xs)
        nb = len(todo)
        uni = rng.random(nb * (D + 1), dtype=np.float32)
        al, out = accept_stochastic(np.asarray(tgt), np.asarray(drf), np.asarray(toks, np.int32),
                                    np.arange(nb + 1, dtype=np.int32) * (D + 1), uni)
        for j, i in enumerate(todo):
            seqs[i].extend(int(v) for v in out[j * (D + 1): j * (D + 1) + al[j]])
    first3 = np.asarray([s[1:4] for s in seqs])
    cell = first3[:, 0] * 16 + first3[:, 1] * 4 + first3[:, 2]
    obs = np.bincount(cell, minlength=64)
    a, b, c = np.meshgrid(np.arange(V), np.arange(V), np.arange(V), indexing="ij")
    joint = (pT[0][a] * pT[a, b] * pT[b, c]).reshape(-1)
    chi = stats.chisquare(obs, joint * N)
    assert chi.pvalue > 1e-4, chi


# ----------------------------------------------------------------------------- acceptance length

def _tau(alpha, gamma):
    return (1 - alpha ** (gamma + 1)) / (1 - alpha)


@pytest.mark.parametrize("alpha", [0.4, 0.6, 0.8])
@pytest.mark.parametrize("D", [3, 7])
def test_mean_acceptance_length_matches_tau(alpha, D):
    spec = preset("g8_kv32k_sweep", batch=500, kv_heads=1, group=1, head_dim=16, kv_len=64,
                  draft_len=D, vocab=2000, alpha=alpha, seed=D * 10 + int(alpha * 10))
    inp = generate(spec)
    al, out = accept_stochastic(**accept_args(inp))
    assert al.min() >= 1 and al.max() <= D + 1
    k = np.arange(1, D + 2)
    pmf = np.where(k <= D, alpha ** (k - 1) * (1 - alpha), alpha ** D)     # truncated geometric
    mean = float((k * pmf).sum())
    assert abs(mean - _tau(alpha, D)) < 1e-12
    var = float((k * k * pmf).sum()) - mean ** 2
    z = (al.mean() - mean) / math.sqrt(var / len(al))
    assert abs(z) < 4.0, (al.mean(), mean, z)
    obs = np.bincount(al, minlength=D + 2)[1:]
    chi = stats.chisquare(obs, pmf * len(al))
    assert chi.pvalue > 1e-4, chi


def test_identical_distributions_accept_everything():
    spec = preset("tiny", batch=6, draft_len=5, seed=3)
    inp = generate(spec)
    args = accept_args(inp)
    qs = args["q_start"]
    args["draft_logits"] = np.concatenate(
        [args["target_logits"][qs[b]:qs[b + 1] - 1] for b in range(len(qs) - 1)])
    al, out = accept_stochastic(**args)
    assert np.all(al == 6)
    tok = args["draft_tokens"]
    for b in range(6):
        assert list(out[qs[b]:qs[b] + 5]) == list(tok[b * 5:(b + 1) * 5])


def test_zero_probability_cases():
    V = 6
    t = np.zeros((2, V), np.float32)
    d = np.zeros((1, V), np.float32)
    qs = np.asarray([0, 2], np.int32)
    t0 = t.copy()
    t0[0, 2] = -np.inf                                   # p(x) = 0 -> reject whatever u is
    al, out = accept_stochastic(t0, d, np.asarray([2], np.int32), qs, np.asarray([0.0, 0.3], np.float32))
    assert al[0] == 1 and out[0] != 2
    d0 = d.copy()
    d0[0, 3] = -np.inf                                   # q(x) = 0 < p(x) -> accept whatever u is
    al, out = accept_stochastic(t, d0, np.asarray([3], np.int32), qs,
                                np.asarray([np.float32(1 - 2**-24), 0.3], np.float32))
    assert al[0] == 2 and out[0] == 3
    both = t0.copy()
    d1 = d.copy()
    d1[0, 2] = -np.inf                                   # p(x) = q(x) = 0 -> reject
    al, out = accept_stochastic(both, d1, np.asarray([2], np.int32), qs, np.asarray([0.0, 0.3], np.float32))
    assert al[0] == 1
    for bad in (-1, V):                                  # out-of-range draft ids fail
        al, out = accept_stochastic(t, d, np.asarray([bad], np.int32), qs, np.asarray([0.0, 0.3], np.float32))
        assert al[0] == 1 and 0 <= out[0] < V


def test_acceptance_length_range_random_inputs():
    for seed in range(4):
        inp = generate(preset("tiny", batch=16, draft_len=(0, 1, 4, 9), seed=seed))
        args = accept_args(inp)
        al, out = accept_stochastic(**args)
        D = np.diff(args["q_start"]) - 1
        assert np.all(al >= 1) and np.all(al <= D + 1)
        for b in range(16):
            seg = out[args["q_start"][b]:args["q_start"][b + 1]]
            assert np.all(seg[:al[b]] >= 0) and np.all(seg[al[b]:] == -1)
        alg, outg = accept_greedy(args["target_logits"], args["draft_tokens"], args["q_start"])
        assert np.all(alg >= 1) and np.all(alg <= D + 1)
