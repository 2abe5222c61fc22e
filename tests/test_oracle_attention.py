"""Pins for the oracle's causal softmax attention (forward and backward).

Closed forms: with Q = 0 every allowed key gets the same weight, so O_i is the
mean of V_0..V_i and LSE_i = log(i+1); row 0 always returns V_0.  Causality:
changing keys/values after row i leaves row i unchanged.  Backward: central
differences of l = sum(O * dO).
"""
import numpy as np

from oracle import stage as ost


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_uniform_attention_closed_form():
    s, d = 9, 4
    q = np.zeros((s, d))
    k = _rand((s, d), 1)
    v = _rand((s, d), 2)
    o, p, lse = ost.causal_attention_forward(q, k, v)
    for i in range(s):
        assert np.allclose(o[i], v[: i + 1].mean(axis=0), atol=1e-14)
        assert abs(lse[i] - np.log(i + 1)) < 1e-14
    assert np.allclose(np.triu(p, 1), 0)


def test_first_row_and_causality():
    s, d = 8, 4
    q, k, v = _rand((s, d), 3), _rand((s, d), 4), _rand((s, d), 5)
    o, _, _ = ost.causal_attention_forward(q, k, v)
    assert np.allclose(o[0], v[0], atol=1e-15)
    k2, v2 = k.copy(), v.copy()
    k2[5:] += 3.0
    v2[5:] -= 2.0
    o2, _, _ = ost.causal_attention_forward(q, k2, v2)
    assert np.array_equal(o[:5], o2[:5])
    assert not np.allclose(o[5:], o2[5:])


def test_softmax_rows_sum_to_one_and_lse():
    s, d = 7, 3
    q, k, v = _rand((s, d), 6), _rand((s, d), 7), _rand((s, d), 8)
    _, p, lse = ost.causal_attention_forward(q, k, v)
    assert np.allclose(p.sum(axis=1), 1.0, atol=1e-14)
    sc = q @ k.T / np.sqrt(d)
    for i in range(s):
        assert abs(lse[i] - np.log(np.exp(sc[i, : i + 1]).sum())) < 1e-13


def test_attention_backward_central_differences():
    s, d = 6, 4
    q, k, v = _rand((s, d), 9), _rand((s, d), 10), _rand((s, d), 11)
    do = _rand((s, d), 12)
    _, p, _ = ost.causal_attention_forward(q, k, v)
    dq, dk, dv = ost.causal_attention_backward(q, k, v, p, do)

    def loss(q_, k_, v_):
        return float((ost.causal_attention_forward(q_, k_, v_)[0] * do).sum())

    eps = 1e-6
    for which, grad in ((0, dq), (1, dk), (2, dv)):
        num = np.zeros_like(grad)
        for i in range(s):
            for j in range(d):
                args_p = [q.copy(), k.copy(), v.copy()]
                args_m = [q.copy(), k.copy(), v.copy()]
                args_p[which][i, j] += eps
                args_m[which][i, j] -= eps
                num[i, j] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
        assert np.max(np.abs(num - grad)) <= 1e-6 * max(1.0, np.max(np.abs(grad)))
