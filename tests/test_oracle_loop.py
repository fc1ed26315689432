"""Pins of the closed-loop oracle (oracle/loop.py): lossless against plain
greedy decoding of the toy LM, the n-gram drafter and the tier rule on hand
cases, full acceptance on a periodic target, and the length cap."""

import numpy as np
import pytest

from oracle.loop import closed_loop, greedy_decode, next_tier, ngram_draft


def _bigram(V, seed, std=3.0):
    return (np.random.default_rng(seed).standard_normal((V, V)) * std).astype(np.float32)


@pytest.mark.parametrize("ngram", [1, 2, 3])
@pytest.mark.parametrize("tiers", [(1, 3, 7), (2,), (0, 4)])
def test_loop_output_is_plain_greedy_decoding(ngram, tiers):
    V = 97
    W = _bigram(V, ngram)
    rng = np.random.default_rng(7)
    hist = [list(rng.integers(0, V, size=int(L))) for L in (1, 5, 30, 64)]
    out, al, d = closed_loop(W, hist, tiers, ngram, 0.5, steps=25, max_len=10_000)
    for h0, h in zip(hist, out):
        assert h[:len(h0)] == h0
        assert h[len(h0):] == greedy_decode(W, h0, len(h) - len(h0))
    assert np.all(al >= 1) and np.all(al <= 1 + d[:, None])
    assert set(d.tolist()) <= set(tiers)


def test_ngram_drafter_by_hand():
    assert ngram_draft([1, 2, 3, 1, 2], 2, 3) == [3, 1, 2]          # suffix (1, 2) at 0
    assert ngram_draft([1, 2, 3, 1, 2], 2, 5) == [3, 1, 2, -1, -1]  # runs out of history
    assert ngram_draft([5, 1, 9, 1, 2, 7, 1], 3, 2) == [2, 7]       # (.., 7, 1) absent: falls back to (1): latest at 3
    assert ngram_draft([4, 8, 6], 2, 2) == [-1, -1]                 # no earlier occurrence of any suffix
    assert ngram_draft([3], 3, 2) == [-1, -1]
    assert ngram_draft([2, 2, 2], 1, 3) == [2, -1, -1]              # latest earlier (2) is at 1: one token follows


def test_tier_rule_by_hand():
    tiers = (1, 3, 7)
    assert [next_tier(e, tiers) for e in (1.0, 1.01, 2.9, 3.0, 3.5, 7.0, 9.0)] == [1, 3, 3, 3, 7, 7, 7]


def test_periodic_target_climbs_to_the_top_tier():
    """A target whose greedy path cycles through 0..p-1: once a cycle is in the
    history the drafter is always right as far as the history reaches (one
    period back), AL = 1 + min(D, p), and the tiers climb."""
    V, p = 64, 5
    W = np.zeros((V, V), np.float32)
    for a in range(V):
        W[a, (a + 1) % p] = 10.0
    hist = [[40, 41, 42, 43], [7, 30]]
    out, al, d = closed_loop(W, hist, (1, 3, 7), 2, 0.5, steps=30, max_len=10_000)
    assert d[0] == 1 and d[-1] == 7
    late = slice(10, 30)
    assert np.all(al[late] == 1 + np.minimum(d[late], p)[:, None])
    for h0, h in zip(hist, out):
        assert h[len(h0):] == greedy_decode(W, h0, len(h) - len(h0))


def test_length_cap():
    V = 31
    W = _bigram(V, 3)
    out, al, _ = closed_loop(W, [[1, 2, 3]], (3,), 1, 0.5, steps=40, max_len=20)
    assert len(out[0]) <= 20
    assert np.all(al[-5:] == 0)
    assert out[0][3:] == greedy_decode(W, [1, 2, 3], len(out[0]) - 3)
