"""Pins for oracle.linear (y = x w^T over token rows): brute force with
math.fsum, closed forms (identity weights copy the rows, a one-hot weight row
picks one input feature, a ones row sums the features), linearity in x, and
a planted-mistake check (transposed operand, dropped term, wrong sign)."""
import math

import numpy as np
import pytest

from oracle import linear as L


def rnd(rng, *shape):
    return rng.standard_normal(shape)


@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (3, 5, 7), (9, 4, 16), (17, 33, 8)])
def test_brute_force(M, N, K):
    rng = np.random.default_rng(M * 1000 + N * 10 + K)
    x, w = rnd(rng, M, K), rnd(rng, N, K)
    want = np.array([[math.fsum(x[t, k] * w[n, k] for k in range(K)) for n in range(N)] for t in range(M)])
    np.testing.assert_allclose(L.linear(x, w), want, rtol=0, atol=1e-13)


def test_identity_weight_copies_rows():
    x = np.random.default_rng(1).standard_normal((6, 12))
    assert np.array_equal(L.linear(x, np.eye(12)), x)


def test_one_hot_and_ones_rows():
    rng = np.random.default_rng(2)
    x = rnd(rng, 5, 10)
    w = np.zeros((3, 10))
    w[0, 7] = 1.0
    w[1, 2] = -1.0
    w[2, :] = 1.0
    y = L.linear(x, w)
    assert np.array_equal(y[:, 0], x[:, 7])
    assert np.array_equal(y[:, 1], -x[:, 2])
    np.testing.assert_allclose(y[:, 2], [math.fsum(r) for r in x], atol=1e-14)


def test_linear_in_x():
    rng = np.random.default_rng(3)
    a, b, w = rnd(rng, 4, 9), rnd(rng, 4, 9), rnd(rng, 6, 9)
    np.testing.assert_allclose(L.linear(2.5 * a - b, w), 2.5 * L.linear(a, w) - L.linear(b, w), atol=1e-12)


def test_shape_errors():
    with pytest.raises(ValueError):
        L.linear(np.zeros((2, 3)), np.zeros((3, 2)))


def _mutant(kind):
    def f(x, w):
        x, w = np.asarray(x, float), np.asarray(w, float)
        if kind == "transposed":          # w used as [K, N]: raises or gives wrong values
            return x @ w
        if kind == "dropped":
            return x[:, 1:] @ w[:, 1:].T
        return -(x @ w.T)
    return f


@pytest.mark.parametrize("kind", ["transposed", "dropped", "sign"])
def test_pins_catch_planted_mistakes(kind, monkeypatch):
    monkeypatch.setattr(L, "linear", _mutant(kind))
    caught = 0
    for pin in [lambda: test_brute_force(3, 5, 7), test_one_hot_and_ones_rows, test_identity_weight_copies_rows]:
        try:
            pin()
        except (AssertionError, ValueError):
            caught += 1
    assert caught >= 1
