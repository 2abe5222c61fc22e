"""Planted mistakes: each test swaps one plausible error into the oracle (on
the CPU, for this test only) and checks that a pin from the other oracle test
files rejects it.  A pin that still passed with the mistake would not be
pinning anything."""
import numpy as np
import pytest

import test_oracle_attention as pin_attn
import test_oracle_elementwise as pin_gelu
import test_oracle_schedules as pin_sched
from oracle import schedules as sch
from oracle import stage as ost


def _attention_forward(scale_of_d, causal=True):
    def forward(q, k, v):
        s, d = q.shape
        scores = (q @ k.T) * scale_of_d(d)
        if causal:
            scores = np.where(np.triu(np.ones((s, s), dtype=bool), k=1), -np.inf, scores)
        row_max = scores.max(axis=1, keepdims=True)
        e = np.exp(scores - row_max)
        denom = e.sum(axis=1, keepdims=True)
        return (e / denom) @ v, e / denom, (row_max + np.log(denom))[:, 0]
    return forward


def test_attention_without_causal_mask_is_caught(monkeypatch):
    monkeypatch.setattr(ost, "causal_attention_forward", _attention_forward(lambda d: 1 / np.sqrt(d), causal=False))
    with pytest.raises(AssertionError):
        pin_attn.test_first_row_and_causality()


def test_attention_with_wrong_scale_is_caught(monkeypatch):
    monkeypatch.setattr(ost, "causal_attention_forward", _attention_forward(lambda d: 1.0 / d))
    with pytest.raises(AssertionError):
        pin_attn.test_softmax_rows_sum_to_one_and_lse()


def test_attention_backward_untransposed_dk_is_caught(monkeypatch):
    def backward(q, k, v, p, do):
        d = q.shape[1]
        dp = do @ v.T
        ds = p * (dp - (dp * p).sum(axis=1, keepdims=True))
        return (ds @ k) / np.sqrt(d), (ds @ q) / np.sqrt(d), p.T @ do  # dK should use ds^T
    monkeypatch.setattr(ost, "causal_attention_backward", backward)
    with pytest.raises(AssertionError):
        pin_attn.test_attention_backward_central_differences()


def test_attention_backward_without_row_correction_is_caught(monkeypatch):
    def backward(q, k, v, p, do):
        d = q.shape[1]
        ds = p * (do @ v.T)  # drops the - rowsum(dP * P) term of the softmax Jacobian
        return (ds @ k) / np.sqrt(d), (ds.T @ q) / np.sqrt(d), p.T @ do
    monkeypatch.setattr(ost, "causal_attention_backward", backward)
    with pytest.raises(AssertionError):
        pin_attn.test_attention_backward_central_differences()


def _zbh1_holding_back(extra):
    def order(P, m, s):
        warm = min(m, P - 1 - s)
        ops = [("F", j) for j in range(warm)]
        next_f, next_w = warm, 0
        for b in range(m):
            if next_f < m:
                ops.append(("F", next_f))
                next_f += 1
            ops.append(("B", b))
            if b >= s + extra:
                ops.append(("W", next_w))
                next_w += 1
        return ops + [("W", j) for j in range(next_w, m)]
    return order


def test_zbh1_holding_back_one_w_too_many_is_caught(monkeypatch):
    bad = _zbh1_holding_back(1)
    monkeypatch.setattr(sch, "order_zbh1", bad)
    monkeypatch.setitem(sch.ORDERS, "zbh1", bad)
    with pytest.raises(AssertionError):
        pin_sched.test_peak_memory_closed_forms(4, 7, 5)


def test_zbh1_with_w_right_after_its_b_is_caught(monkeypatch):
    bad = _zbh1_holding_back(-10 ** 6)  # every W right after its own B: 1F1B's bubble
    monkeypatch.setattr(sch, "order_zbh1", bad)
    monkeypatch.setitem(sch.ORDERS, "zbh1", bad)
    with pytest.raises(AssertionError):
        pin_sched.test_table2_bubble_closed_forms(4, (2, 3, 1))


def test_zbh2_with_one_warmup_forward_too_many_is_caught(monkeypatch):
    good = sch.order_zbh2

    def bad(P, m, s):
        ops = good(P, m, s)
        first_b = next(i for i, (k, _) in enumerate(ops) if k == "B")
        if first_b < len(ops) and any(k == "F" for k, _ in ops[first_b:]):
            i = next(i for i in range(first_b, len(ops)) if ops[i][0] == "F")
            ops.insert(first_b, ops.pop(i))  # one more forward before the first B
        return ops
    monkeypatch.setattr(sch, "order_zbh2", bad)
    monkeypatch.setitem(sch.ORDERS, "zbh2", bad)
    with pytest.raises(AssertionError):
        pin_sched.test_zbh2_first_stage_runs_seven_forwards_before_first_b()


def test_heuristic_memory_check_off_by_one_microbatch_is_caught(monkeypatch):
    import test_oracle_heuristic as pin_heur
    from oracle import heuristic as H
    good = H.build

    def bad(P, m, t, m_b, m_w, m_limit, *args, **kw):  # checks against one activation more than allowed
        return good(P, m, t, m_b, m_w, m_limit + m_b, *args, **kw)
    monkeypatch.setattr(H, "build", bad)
    with pytest.raises(AssertionError):
        for seed in range(6):
            pin_heur.test_orders_valid_and_within_budget(seed)


def test_v_placement_as_a_ring_is_caught(monkeypatch):
    import test_oracle_vshape as pin_v
    from oracle import vshape as V
    monkeypatch.setattr(V, "device_of", lambda c, P: c % P)  # interleaved placement instead of the V
    with pytest.raises(AssertionError):
        pin_v.test_placement_is_a_v(2)


@pytest.mark.parametrize("a", [0.0, 0.04715])
def test_gelu_tanh_without_or_with_a_mistyped_cubic_term_is_caught(monkeypatch, a):
    monkeypatch.setattr(ost, "_TANH_A", a)
    with pytest.raises(AssertionError):
        pin_gelu.test_gelu_tanh_stays_within_the_approximation_band_of_exact_gelu()


def test_gelu_tanh_grad_without_the_chain_factor_is_caught(monkeypatch):
    def grad(z, form="erf"):
        t = np.tanh(ost._TANH_C * (z + ost._TANH_A * np.asarray(z) ** 3))
        return 0.5 * (1.0 + t) + 0.5 * z * (1.0 - t * t)
    monkeypatch.setattr(ost, "gelu_grad", grad)
    with pytest.raises(AssertionError):
        pin_gelu.test_gelu_tanh_grad_central_differences()
