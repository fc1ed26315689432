"""Pins of the relaxed-acceptance oracle (oracle/lossy.py) against library
routines, closed forms and the lossless oracle."""

import math

import numpy as np
import pytest
from scipy.spatial.distance import jensenshannon
from scipy.stats import entropy

from oracle import accept_greedy, accept_lossy, accept_stochastic, js_distance, row_entropy
from workloads import WorkloadSpec, generate


def _softmax(x):
    x = np.asarray(x, np.float64)
    e = np.exp(x - x.max())
    return e / e.sum()


def test_statistics_match_scipy():
    rng = np.random.default_rng(0)
    for V in (2, 7, 1000):
        for _ in range(5):
            t = rng.standard_normal(V) * 3
            d = t + rng.standard_normal(V)
            assert abs(js_distance(t, d) - jensenshannon(_softmax(t), _softmax(d))) < 1e-12
            assert abs(row_entropy(d) - entropy(_softmax(d))) < 1e-12


def test_closed_forms():
    V = 64
    # identical rows: distance 0; uniform rows: entropy ln V
    x = np.random.default_rng(1).standard_normal(V)
    assert js_distance(x, x) == pytest.approx(0.0, abs=1e-7)
    assert row_entropy(np.zeros(V)) == pytest.approx(math.log(V), abs=1e-12)
    # one-hot row: entropy 0
    oh = np.full(V, -np.inf)
    oh[5] = 0.0
    assert row_entropy(oh) == 0.0
    # disjoint supports: JSD = ln 2
    a = np.full(V, -np.inf)
    a[:32] = 0.0
    b = np.full(V, -np.inf)
    b[32:] = 0.0
    assert js_distance(a, b) == pytest.approx(math.sqrt(math.log(2)), abs=1e-12)
    # two tokens: p = (s, 1-s), q = (r, 1-r) written out by hand
    s, r = 0.8, 0.3
    m0, m1 = (s + r) / 2, (2 - s - r) / 2
    jsd = 0.5 * (s * math.log(s / m0) + (1 - s) * math.log((1 - s) / m1)) + \
        0.5 * (r * math.log(r / m0) + (1 - r) * math.log((1 - r) / m1))
    assert js_distance(np.log([s, 1 - s]), np.log([r, 1 - r])) == pytest.approx(math.sqrt(jsd), abs=1e-12)
    # symmetric
    y = np.random.default_rng(2).standard_normal(V)
    assert js_distance(x, y) == pytest.approx(js_distance(y, x), abs=1e-14)


def _inputs(mode, seed, vocab=300, draft_noise_std=1.0):
    return generate(WorkloadSpec(name="lossy", batch=6, kv_heads=1, group=1, head_dim=64, kv_len=64,
                                 draft_len=[0, 1, 3, 7, 5, 2], vocab=vocab, mode="stochastic", target_std=2.0,
                                 draft_noise_std=draft_noise_std, seed=seed))


def _args(inp):
    return dict(target_logits=inp.target_logits.numpy(), draft_logits=inp.draft_logits.numpy(),
                draft_tokens=inp.draft_tokens.numpy(), q_start=inp.q_start.numpy(), uniforms=inp.uniforms.numpy())


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_negative_threshold_is_the_lossless_rule(seed):
    inp = _inputs("stochastic", seed)
    a = _args(inp)
    al, out, ent, js = accept_lossy("stochastic", js_threshold=-1.0, **a)
    al0, out0 = accept_stochastic(**a)
    assert np.array_equal(al, al0) and np.array_equal(out, out0)
    al, out, _, _ = accept_lossy("greedy", js_threshold=-1.0, **a)
    al0, out0 = accept_greedy(a["target_logits"], a["draft_tokens"], a["q_start"])
    assert np.array_equal(al, al0) and np.array_equal(out, out0)
    # statistics of every drafted row, whatever the decisions
    d0 = 0
    qs = a["q_start"]
    for b in range(len(qs) - 1):
        t0 = int(qs[b])
        for i in range(int(qs[b + 1]) - t0 - 1):
            assert ent[d0] == pytest.approx(entropy(_softmax(a["draft_logits"][d0])), abs=1e-10)
            assert js[d0] == pytest.approx(jensenshannon(_softmax(a["target_logits"][t0 + i]),
                                                         _softmax(a["draft_logits"][d0])), abs=1e-10)
            d0 += 1


@pytest.mark.parametrize("mode", ["greedy", "stochastic"])
def test_threshold_at_the_maximum_accepts_every_valid_draft(mode):
    inp = _inputs(mode, 3)
    a = _args(inp)
    qs = a["q_start"]
    tokens = a["draft_tokens"].copy()
    tokens[4] = -1                                   # sequence 3 (drafts at 4..10) stops at its 1st draft...
    a["draft_tokens"] = tokens
    al, out, _, _ = accept_lossy(mode, js_threshold=math.sqrt(math.log(2)) + 1e-9, **a)
    D = np.diff(qs) - 1
    expect = 1 + D
    # the sequence holding the out-of-range token stops there
    d0s = qs[:-1] - np.arange(len(D))
    for b in range(len(D)):
        if d0s[b] <= 4 < d0s[b] + D[b]:
            expect[b] = 1 + (4 - d0s[b])
    assert np.array_equal(al, expect)
    for b in range(len(D)):
        t0 = int(qs[b])
        assert np.array_equal(out[t0:t0 + al[b] - 1], tokens[d0s[b]:d0s[b] + al[b] - 1])


@pytest.mark.parametrize("mode", ["greedy", "stochastic"])
def test_acceptance_grows_with_the_threshold(mode):
    inp = _inputs(mode, 4, draft_noise_std=0.7)
    a = _args(inp)
    prev = None
    for tau in (-1.0, 0.05, 0.1, 0.2, 0.3, 0.5, 0.9):
        al, _, _, _ = accept_lossy(mode, js_threshold=tau, **a)
        if prev is not None:
            assert np.all(al >= prev)
        prev = al


def test_relaxed_position_takes_the_draft_token():
    """One sequence, two drafts: the lossless test fails at draft 1 (u above
    p/q), the JS distance of its rows is below tau, so it passes; draft 2 fails
    both and is resampled from the residual at row 2."""
    V = 4
    # (logits are fp32, as the call takes them)
    t = np.log(np.array([[0.4, 0.3, 0.2, 0.1], [0.1, 0.2, 0.3, 0.4], [0.25, 0.25, 0.25, 0.25]])).astype(np.float32)
    d = np.log(np.array([[0.45, 0.25, 0.2, 0.1], [0.7, 0.1, 0.1, 0.1]])).astype(np.float32)
    tokens = np.array([0, 0])                      # p/q = 0.4/0.45 at row 0, 0.1/0.7 at row 1
    u = np.array([0.95, 0.9, 0.5], np.float32)
    qs = np.array([0, 3])
    js0 = jensenshannon(_softmax(t[0]), _softmax(d[0]))
    js1 = jensenshannon(_softmax(t[1]), _softmax(d[1]))
    assert js0 < 0.1 < js1
    al, out, _, js = accept_lossy("stochastic", t, d, tokens, qs, u, js_threshold=0.1)
    assert al[0] == 2 and out[0] == 0 and out[2] == -1
    # residual max(0, p - q) at row 1 = (0, 0.1, 0.2, 0.3): u = 0.5 of 0.6 falls on token 2
    assert out[1] == 2
    assert js[0] == pytest.approx(js0, abs=1e-12) and js[1] == pytest.approx(js1, abs=1e-12)
    al, out, _, _ = accept_lossy("stochastic", t, d, tokens, qs, u, js_threshold=-1)
    assert al[0] == 1
