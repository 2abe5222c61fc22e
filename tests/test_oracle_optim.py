"""Pins of the optimizer oracle (oracle/optim.py): AdamW and gradient clipping
against PyTorch's own CPU implementations in fp64, the exact inverse
(rollback) of a step, and the post-update validation protocol against the
synchronous step it replaces ("Zero Bubble Pipeline Parallelism", section 4
and Appendix C)."""
import numpy as np
import pytest
import torch

from oracle import optim as O

HP = O.AdamW(lr=1e-2, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.1, max_grad_norm=1.0)


def _tensors(rng, shapes, scale=1.0):
    return [rng.standard_normal(s) * scale for s in shapes]


def test_adamw_matches_torch():
    rng = np.random.default_rng(0)
    shapes = [(3, 5), (7,)]
    theta = _tensors(rng, shapes)
    tp = [torch.tensor(t, dtype=torch.float64, requires_grad=True) for t in theta]
    opt = torch.optim.AdamW(tp, lr=HP.lr, betas=(HP.beta1, HP.beta2), eps=HP.eps, weight_decay=HP.weight_decay)
    m = [np.zeros(s) for s in shapes]
    v = [np.zeros(s) for s in shapes]
    for step in range(1, 4):
        grads = _tensors(rng, shapes)
        for p, g in zip(tp, grads):
            p.grad = torch.tensor(g)
        opt.step()
        for i in range(len(shapes)):
            theta[i], m[i], v[i] = O.adamw_step(theta[i], m[i], v[i], grads[i], 1.0, step, HP)
            np.testing.assert_allclose(theta[i], tp[i].detach().numpy(), rtol=1e-13, atol=1e-15)
            st = opt.state[tp[i]]
            np.testing.assert_allclose(m[i], st["exp_avg"].numpy(), rtol=1e-13, atol=1e-15)
            np.testing.assert_allclose(v[i], st["exp_avg_sq"].numpy(), rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("scale", [1e-3, 10.0])
def test_clip_matches_torch(scale):
    rng = np.random.default_rng(1)
    grads = _tensors(rng, [(4, 6), (9,)], scale)
    tp = [torch.zeros(g.shape, dtype=torch.float64, requires_grad=True) for g in grads]
    for p, g in zip(tp, grads):
        p.grad = torch.tensor(g)
    torch.nn.utils.clip_grad_norm_(tp, HP.max_grad_norm)
    coef = O.clip_coef(O.local_state(grads), HP)
    for p, g in zip(tp, grads):
        np.testing.assert_allclose(coef * g, p.grad.numpy(), rtol=1e-14)
    assert (coef == 1.0) == (scale < 1)


def test_nonfinite_skips_the_step():
    g = np.array([1.0, np.nan])
    assert O.local_state([g])[1] is True
    assert O.clip_coef(O.local_state([g]), HP) is None
    th, m, v = O.adamw_step(np.ones(2), np.zeros(2), np.zeros(2), g, None, 1, HP)
    assert np.array_equal(th, np.ones(2)) and not m.any() and not v.any()


def test_rollback_inverts_a_step():
    rng = np.random.default_rng(2)
    theta, m, v = rng.standard_normal(64), rng.standard_normal(64) * 0.1, rng.random(64) * 0.01
    for step in (1, 2, 7):
        for coef in (1.0, 0.37):
            g = rng.standard_normal(64)
            th1, m1, v1 = O.adamw_step(theta, m, v, g, coef, step, HP)
            th0, m0, v0 = O.adamw_rollback(th1, m1, v1, g, coef, step, HP)
            np.testing.assert_allclose(th0, theta, rtol=1e-12, atol=1e-15)
            np.testing.assert_allclose(m0, m, rtol=1e-9, atol=1e-15)
            np.testing.assert_allclose(v0, v, rtol=1e-9, atol=1e-15)


def test_rollback_is_bit_exact_on_dyadic_values():
    """With dyadic hyperparameters and gradients whose moments have exact square
    roots, every operation of the step and of its inverse is exact."""
    hp = O.AdamW(lr=0.25, beta1=0.5, beta2=0.5, eps=0.0, weight_decay=0.0, max_grad_norm=0.0)
    theta = np.array([1.0, -2.0, 0.5, 3.0])
    g = np.array([1.0, -2.0, 4.0, 0.5])
    th1, m1, v1 = O.adamw_step(theta, np.zeros(4), np.zeros(4), g, 1.0, 1, hp)
    assert np.array_equal(th1, theta - 0.25 * np.sign(g))
    th0, m0, v0 = O.adamw_rollback(th1, m1, v1, g, 1.0, 1, hp)
    assert np.array_equal(th0, theta) and not m0.any() and not v0.any()


def test_planted_rollback_mistake_is_caught():
    """Dropping the weight-decay factor from the inverse breaks the round trip."""
    rng = np.random.default_rng(3)
    theta, g = rng.standard_normal(16), rng.standard_normal(16)
    th1, m1, v1 = O.adamw_step(theta, np.zeros(16), np.zeros(16), g, 1.0, 1, HP)
    mhat, vhat = m1 / (1 - HP.beta1), v1 / (1 - HP.beta2)
    wrong = th1 + HP.lr * mhat / (np.sqrt(vhat) + HP.eps)
    assert not np.allclose(wrong, theta, rtol=1e-6)


def _pipeline(rng, P, scales, nan_stage=None):
    shapes = [(5, 3), (6,)]
    params = [_tensors(rng, shapes) for _ in range(P)]
    moms = [_tensors(rng, shapes, 0.01) for _ in range(P)]
    vels = [[np.abs(x) * 1e-3 for x in _tensors(rng, shapes)] for _ in range(P)]
    grads = [_tensors(rng, shapes, scales[s]) for s in range(P)]
    if nan_stage is not None:
        grads[nan_stage][0][0, 0] = np.inf
    return params, moms, vels, grads


@pytest.mark.parametrize("case", ["no_clip", "clip_late", "clip_all", "nonfinite_last"])
def test_post_validated_step_equals_synchronous(case):
    P = 4
    rng = np.random.default_rng(4)
    scales = {"no_clip": [0.01] * P, "clip_late": [0.01, 0.01, 0.01, 1.0], "clip_all": [1.0] * P,
              "nonfinite_last": [0.01] * P}[case]
    params, moms, vels, grads = _pipeline(rng, P, scales, nan_stage=3 if case == "nonfinite_last" else None)
    step = 3
    p1, m1, v1, rolled = O.post_validated_step(params, moms, vels, grads, step, HP)
    p2, m2, v2 = O.synchronous_step(params, moms, vels, grads, step, HP)
    for s in range(P):
        for a, b in zip(p1[s] + m1[s] + v1[s], p2[s] + m2[s] + v2[s]):
            np.testing.assert_allclose(a, b, rtol=1e-10, atol=1e-14)
    assert rolled[-1] is False                       # the last stage steps with the global state
    expect = {"no_clip": [False] * P, "clip_late": [True, True, True, False],
              "clip_all": [True, True, True, False], "nonfinite_last": [True, True, True, False]}[case]
    assert rolled == expect
    if case == "nonfinite_last":                     # nothing moved anywhere
        for s in range(P):
            for a, b in zip(p1[s], params[s]):
                np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-15)


def test_synchronous_step_matches_torch_clip_and_adamw():
    rng = np.random.default_rng(5)
    P = 3
    params, moms, vels, grads = _pipeline(rng, P, [1.0] * P)
    flat = [t for s in range(P) for t in params[s]]
    tp = [torch.tensor(t, dtype=torch.float64, requires_grad=True) for t in flat]
    opt = torch.optim.AdamW(tp, lr=HP.lr, betas=(HP.beta1, HP.beta2), eps=HP.eps, weight_decay=HP.weight_decay)
    zeros = [[np.zeros_like(t) for t in params[s]] for s in range(P)]
    for p, g in zip(tp, [g for s in range(P) for g in grads[s]]):
        p.grad = torch.tensor(g)
    torch.nn.utils.clip_grad_norm_(tp, HP.max_grad_norm)
    opt.step()
    p2, _, _ = O.synchronous_step(params, zeros, zeros, grads, 1, HP)
    for a, b in zip([t for s in range(P) for t in p2[s]], tp):
        np.testing.assert_allclose(a, b.detach().numpy(), rtol=1e-12, atol=1e-15)
