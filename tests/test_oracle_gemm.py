"""Pins of the verify-linear oracle against things other than itself.

* closed forms: an identity weight returns x; a permutation weight returns the
  permuted columns of x (the direction of the permutation fixes which operand
  is transposed); an all-ones row of x returns the row sums of W; a diagonal
  weight scales the columns;
* brute force: on a tiny case, every element equals the sum over k written out
  with Python floats;
* shapes: y is [M, N] for x [M, K] and W [N, K], and mismatched K is refused.
"""

import numpy as np
import pytest

from oracle import linear_abs_sum, verify_linear


def _bf16_bits(a):
    """fp32 values -> bf16 bit patterns (round to nearest even)."""
    u = np.asarray(a, np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def _from_bits(b):
    return (np.asarray(b).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def test_identity_weight_returns_x():
    rng = np.random.default_rng(0)
    x = _bf16_bits(rng.standard_normal((5, 64)))
    w = _bf16_bits(np.eye(64))
    np.testing.assert_array_equal(verify_linear(x, w), _from_bits(x))


def test_permutation_weight_permutes_columns():
    rng = np.random.default_rng(1)
    K = 64
    perm = np.roll(np.arange(K), 5)            # not an involution: the two operand orders differ
    wm = np.zeros((K, K))
    wm[np.arange(K), perm] = 1.0               # row n of W picks input feature perm[n]
    x = _bf16_bits(rng.standard_normal((3, K)))
    y = verify_linear(x, _bf16_bits(wm))
    np.testing.assert_array_equal(y, _from_bits(x)[:, perm])
    assert not np.array_equal(y, _from_bits(x)[:, np.argsort(perm)])


def test_ones_row_gives_weight_row_sums():
    rng = np.random.default_rng(2)
    w = _bf16_bits(rng.standard_normal((128, 192)) * 0.25)
    x = _bf16_bits(np.ones((2, 192)))
    y = verify_linear(x, w)
    sums = np.array([sum(float(v) for v in row) for row in _from_bits(w)])
    np.testing.assert_allclose(y[0], sums, rtol=0, atol=1e-12)
    np.testing.assert_array_equal(y[0], y[1])


def test_diagonal_weight_scales_columns():
    rng = np.random.default_rng(3)
    d = _bf16_bits(rng.uniform(-2, 2, 64))
    x = _bf16_bits(rng.standard_normal((4, 64)))
    y = verify_linear(x, _bf16_bits(np.diag(_from_bits(d))))
    np.testing.assert_array_equal(y, _from_bits(x) * _from_bits(d)[None, :])


def test_brute_force_tiny():
    rng = np.random.default_rng(4)
    x = _bf16_bits(rng.standard_normal((3, 8)))
    w = _bf16_bits(rng.standard_normal((5, 8)))
    xf, wf = _from_bits(x), _from_bits(w)
    y = verify_linear(x, w)
    for m in range(3):
        for n in range(5):
            s = 0.0
            for k in range(8):
                s += float(xf[m, k]) * float(wf[n, k])
            assert abs(y[m, n] - s) <= 1e-12 * max(1.0, abs(s))
    assert np.all(linear_abs_sum(x, w) >= np.abs(y) - 1e-12)


def test_abs_sum_brute_force():
    """linear_abs_sum pinned from both sides: Python-float sums of |x w| term by
    term on a tiny case with mixed signs (where |x W^T| is strictly smaller),
    and closed forms (non-negative operands: equal to x W^T; a row of -1
    against ones: K)."""
    rng = np.random.default_rng(5)
    x = _bf16_bits(rng.standard_normal((3, 8)))
    w = _bf16_bits(rng.standard_normal((5, 8)))
    xf, wf = _from_bits(x), _from_bits(w)
    got = linear_abs_sum(x, w)
    assert got.shape == (3, 5)
    for m in range(3):
        for n in range(5):
            s = 0.0
            for k in range(8):
                s += abs(float(xf[m, k]) * float(wf[n, k]))
            assert abs(got[m, n] - s) <= 1e-12 * max(1.0, s)
    assert np.any(got > np.abs(verify_linear(x, w)) + 1e-6)     # cancellation is not counted
    xp = _bf16_bits(np.abs(rng.standard_normal((4, 64))))
    wp = _bf16_bits(np.abs(rng.standard_normal((6, 64))))
    np.testing.assert_allclose(linear_abs_sum(xp, wp), verify_linear(xp, wp), rtol=1e-14)
    ones = _bf16_bits(np.ones((2, 64)))
    neg = _bf16_bits(-np.ones((1, 64)))
    np.testing.assert_array_equal(linear_abs_sum(neg, ones), np.full((1, 2), 64.0))


def test_shapes():
    x = np.zeros((7, 64), np.uint16)
    w = np.zeros((128, 64), np.uint16)
    assert verify_linear(x, w).shape == (7, 128)
    with pytest.raises(ValueError):
        verify_linear(np.zeros((7, 32), np.uint16), w)
