"""Pins for the oracle's linear F/B/W (the split of the backward pass).

Brute force: with small-integer X, W, dY the scalar l = sum(Y * dY) is exact
in fp64, and so are its finite differences l(X + E_ik) - l(X) and
l(W + E_kn) - l(W), which are exactly dX_ik and dW_kn.  l is evaluated with
explicit loops, independent of the oracle's matrix products.  Shapes are
non-square so a transposed operand cannot pass.
"""
import itertools

import numpy as np
import pytest

import synthetic_inputs as si
from oracle import stage as ost


def _loss_loops(x, w, dy):
    t, k = x.shape
    n = w.shape[1]
    total = 0.0
    for a in range(t):
        for c in range(n):
            y = 0.0
            for b in range(k):
                y += x[a, b] * w[b, c]
            total += y * dy[a, c]
    return total


@pytest.mark.parametrize("shape", [(3, 4, 5), (5, 2, 3), (1, 6, 2)])
def test_linear_grads_brute_force_exact(shape):
    t, k, n = shape
    x = si.integer_valued((t, k), -3, 3, seed=1).astype(np.float64)
    w = si.integer_valued((k, n), -3, 3, seed=2).astype(np.float64)
    dy = si.integer_valued((t, n), -3, 3, seed=3).astype(np.float64)
    base = _loss_loops(x, w, dy)
    dx = ost.linear_backward_input(dy, w)
    dw = ost.linear_backward_weight(x, dy)
    assert dx.shape == (t, k) and dw.shape == (k, n)
    for a, b in itertools.product(range(t), range(k)):
        xp = x.copy()
        xp[a, b] += 1.0
        assert _loss_loops(xp, w, dy) - base == dx[a, b]
    for b, c in itertools.product(range(k), range(n)):
        wp = w.copy()
        wp[b, c] += 1.0
        assert _loss_loops(x, wp, dy) - base == dw[b, c]
    y = ost.linear_forward(x, w)
    assert float((y * dy).sum()) == base


def test_planted_transpose_mistake_is_caught():
    """A B pass that forgot the transpose (dY.W on a square W) must fail the brute force."""
    t, k = 3, 3
    x = si.integer_valued((t, k), -3, 3, seed=4).astype(np.float64)
    w = si.integer_valued((k, k), -3, 3, seed=5).astype(np.float64)
    dy = si.integer_valued((t, k), -3, 3, seed=6).astype(np.float64)
    wrong = dy @ w
    base = _loss_loops(x, w, dy)
    diffs = []
    for a, b in itertools.product(range(t), range(k)):
        xp = x.copy()
        xp[a, b] += 1.0
        diffs.append((_loss_loops(xp, w, dy) - base) == wrong[a, b])
    assert not all(diffs)


@pytest.mark.parametrize("m", [2, 5])
def test_deferred_w_sum_equals_full_batch_exact(m):
    """Sum over microbatches of X_j^T dY_j, added in any order, equals the
    full-batch X^T dY exactly (integer inputs keep every fp64 sum exact)."""
    t, k, n = 7, 6, 4
    xs = [si.integer_valued((t, k), -2, 2, seed=10 + j).astype(np.float64) for j in range(m)]
    dys = [si.integer_valued((t, n), -2, 2, seed=20 + j).astype(np.float64) for j in range(m)]
    full = ost.linear_backward_weight(np.concatenate(xs), np.concatenate(dys))
    rng = np.random.default_rng(0)
    for _ in range(6):
        order = rng.permutation(m)
        acc = np.zeros((k, n))
        for j in order:
            acc += ost.linear_backward_weight(xs[j], dys[j])
        assert np.array_equal(acc, full)
