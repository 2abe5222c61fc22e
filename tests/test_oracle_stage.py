"""Pins for the oracle's stage chain (all three layer kinds).

* B and W of a whole stage against central differences of l = sum(y * G).
* The unsplit backward gives the same dx and dW as B followed by W.
* Deferred W: per-microbatch weight gradients summed in any order equal the
  full-batch fused backward ([ZB] section 5, bit-to-bit identity across
  schedules; [AUD] "Split backward without changing the update").
* Table 1 FLOP identities of [ZB] section 2 for the workload accounting.
"""
import numpy as np
import pytest

import synthetic_inputs as si
from oracle import stage as ost

TINY = si.Workload("t", 90, si.TINY_MLP, 2, 4, 12, 0, 5, 1, 3, 2, "zbh1", "fp32")
MLPL = si.Workload("m", 91, si.MLP_LINEARS, 2, 4, 12, 2, 5, 1, 3, 2, "zbh1", "fp32")
FULL = si.Workload("f", 92, si.FULL, 2, 8, 16, 2, 5, 2, 3, 2, "zbh1", "fp32")


def _weights(w, seed, scale=0.5):
    rng = np.random.default_rng(seed)
    return [{nm: scale * rng.standard_normal((k, n)) for nm, k, n in w.linears()}
            for _ in range(w.n_layers)]


def _loss(w, ws, x, g):
    y, _ = ost.stage_forward(w, ws, x)
    return float((y * g).sum())


@pytest.mark.parametrize("w", [TINY, MLPL, FULL], ids=["tiny", "mlp_linears", "full"])
def test_stage_grads_central_differences(w):
    rng = np.random.default_rng(1)
    ws = _weights(w, 2)
    x = rng.standard_normal((w.tokens, w.hidden))
    g = rng.standard_normal((w.tokens, w.hidden))
    y, saved = ost.stage_forward(w, ws, x)
    dx, grads = ost.stage_backward_input(w, ws, saved, g)
    dws = ost.stage_backward_weight(w, saved, grads)
    eps = 1e-6
    picks = [(int(rng.integers(w.tokens)), int(rng.integers(w.hidden))) for _ in range(8)]
    for (i, j) in picks:
        xp, xm = x.copy(), x.copy()
        xp[i, j] += eps
        xm[i, j] -= eps
        num = (_loss(w, ws, xp, g) - _loss(w, ws, xm, g)) / (2 * eps)
        assert abs(num - dx[i, j]) <= 1e-6 * max(1.0, abs(dx[i, j]))
    for li in range(w.n_layers):
        for nm, k, n in w.linears():
            for _ in range(3):
                a, b = int(rng.integers(k)), int(rng.integers(n))
                wp = [{kk: vv.copy() for kk, vv in l.items()} for l in ws]
                wm = [{kk: vv.copy() for kk, vv in l.items()} for l in ws]
                wp[li][nm][a, b] += eps
                wm[li][nm][a, b] -= eps
                num = (_loss(w, wp, x, g) - _loss(w, wm, x, g)) / (2 * eps)
                got = dws[li][nm][a, b]
                assert abs(num - got) <= 1e-6 * max(1.0, abs(got)), (li, nm, a, b)


def test_planted_gelu_derivative_mistake_is_caught(monkeypatch):
    """Swap g' for g inside B: the central-difference pin must fail."""
    w = TINY
    rng = np.random.default_rng(3)
    ws = _weights(w, 4)
    x = rng.standard_normal((w.tokens, w.hidden))
    g = rng.standard_normal((w.tokens, w.hidden))
    monkeypatch.setattr(ost, "gelu_grad", ost.gelu)
    _, saved = ost.stage_forward(w, ws, x)
    dx, _ = ost.stage_backward_input(w, ws, saved, g)
    eps = 1e-6
    xp, xm = x.copy(), x.copy()
    xp[0, 0] += eps
    xm[0, 0] -= eps
    num = (_loss(w, ws, xp, g) - _loss(w, ws, xm, g)) / (2 * eps)
    assert abs(num - dx[0, 0]) > 1e-4


@pytest.mark.parametrize("w", [TINY, MLPL, FULL], ids=["tiny", "mlp_linears", "full"])
def test_split_equals_fused(w):
    rng = np.random.default_rng(5)
    ws = _weights(w, 6)
    x = rng.standard_normal((w.tokens, w.hidden))
    g = rng.standard_normal((w.tokens, w.hidden))
    _, saved = ost.stage_forward(w, ws, x)
    dx_s, grads = ost.stage_backward_input(w, ws, saved, g)
    dw_s = ost.stage_backward_weight(w, saved, grads)
    dx_f, dw_f = ost.stage_backward_fused(w, ws, saved, g)
    assert np.allclose(dx_s, dx_f, rtol=0, atol=1e-12 * np.abs(dx_f).max())
    for a, b in zip(dw_s, dw_f):
        for nm in b:
            assert np.allclose(a[nm], b[nm], rtol=0, atol=1e-12 * np.abs(b[nm]).max())


@pytest.mark.parametrize("w", [TINY, MLPL, FULL], ids=["tiny", "mlp_linears", "full"])
def test_deferred_w_matches_full_batch_fused(w):
    rng = np.random.default_rng(7)
    ws = _weights(w, 8)
    xs = [rng.standard_normal((w.tokens, w.hidden)) for _ in range(w.n_micro)]
    gs = [rng.standard_normal((w.tokens, w.hidden)) for _ in range(w.n_micro)]
    y_full, dx_full, dw_full = ost.stage_full_batch_fused(w, ws, xs, gs)
    for order in ([0, 1, 2], [2, 0, 1], [1, 2, 0]):
        acc = None
        for j in order:
            _, saved = ost.stage_forward(w, ws, xs[j])
            _, grads = ost.stage_backward_input(w, ws, saved, gs[j])
            acc = ost.add_grads(acc, ost.stage_backward_weight(w, saved, grads))
        for a, b in zip(acc, dw_full):
            for nm in b:
                assert np.allclose(a[nm], b[nm], rtol=0, atol=1e-12 * np.abs(b[nm]).max())


def test_pipeline_chains_stages():
    w = MLPL.replace(n_stages=3, n_micro=2)
    wps = [_weights(w, 30 + s) for s in range(w.n_stages)]
    rng = np.random.default_rng(9)
    xs = [rng.standard_normal((w.tokens, w.hidden)) for _ in range(2)]
    gs = [rng.standard_normal((w.tokens, w.hidden)) for _ in range(2)]
    r = ost.pipeline(w, wps, xs, gs)
    for j in range(2):
        y = xs[j]
        for s in range(3):
            y, _ = ost.stage_forward(w, ost.to64(wps[s]), y)
            assert np.array_equal(y, r["y"][s][j])
        # the gradient leaving stage s+1 is the one entering stage s
        _, saved = ost.stage_forward(w, ost.to64(wps[1]), r["y"][0][j])
        dx1, _ = ost.stage_backward_input(w, ost.to64(wps[1]), saved, r["dx"][2][j])
        assert np.array_equal(dx1, r["dx"][1][j])


@pytest.mark.parametrize("name", ["gpt_full_h4096", "gpt_full_h6144", "gpt_full_s4096"])
def test_table1_flop_identities(name):
    """[ZB] Table 1: F = sbh(24h+4s), B = sbh(24h+8s), W = 24sbh^2 per layer, so B + W = 2F.
    Our GEMM count is the 24sbh^2 term; attention is counted causal-only (half of 4s^2bh)."""
    w = si.WORKLOADS[name]
    s, b, h, L = w.seq, w.micro_batch, w.hidden, w.n_layers
    assert w.gemm_flops_per_pass() == L * 24 * s * b * h * h
    assert 2 * w.attn_flops_fwd() == L * 4 * s * s * b * h
    assert 2 * w.attn_flops_bwd() == L * 8 * s * s * b * h
    f = w.gemm_flops_per_pass() + w.attn_flops_fwd()
    bb = w.gemm_flops_per_pass() + w.attn_flops_bwd()
    ww = w.gemm_flops_per_pass()
    assert bb + ww == 2 * f
