"""fp64 oracle of one pipeline stage: F, B, W and the fused backward.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Plain definitions in
numpy float64; a matrix product is the only library primitive used.

Definitions followed
--------------------
* [ZB] section 3 "The Backward Pass Decomposition: B and W": a layer maps
  y = f(x, W); B is the gradient with respect to the layer input, W the
  gradient with respect to the layer's parameters.
* [TUT] "Zero bubble: split the backward pass": for a linear Y = X.W the input
  gradient is dX = dY.W^T and the weight gradient is dW = X^T.dY.
* GeLU (exact, erf form): g(z) = z.Phi(z), g'(z) = Phi(z) + z.phi(z).
* Causal softmax attention per head: S = Q.K^T / sqrt(d) with S_ij = -inf for
  j > i, P = softmax over each row, O = P.V; backward dV = P^T.dO,
  dP = dO.V^T, dS = P * (dP - rowsum(dP * P)), dQ = dS.K / sqrt(d),
  dK = dS^T.Q / sqrt(d).

Stage graphs (readings recorded in the design notes):
* TINY_MLP:    y = GeLU(x.W_up).W_down
* MLP_LINEARS: qkv = x.W_qkv; o = V columns of qkv (identity attention);
               p = o.W_proj; y = GeLU(p.W_up).W_down         (no residual)
* FULL:        x1 = x + Attn(x.W_qkv).W_proj; y = x1 + GeLU(x1.W_up).W_down
"""
from __future__ import annotations

from typing import Dict, List, Sequence

import numpy as np
from scipy.special import erf

import synthetic_inputs as si

_SQRT2 = np.sqrt(2.0)
_INV_SQRT_2PI = 1.0 / np.sqrt(2.0 * np.pi)


# ---------------------------------------------------------------- elementwise

def normal_cdf(z):
    return 0.5 * (1.0 + erf(np.asarray(z, dtype=np.float64) / _SQRT2))


def normal_pdf(z):
    z = np.asarray(z, dtype=np.float64)
    return _INV_SQRT_2PI * np.exp(-0.5 * z * z)


_TANH_C = np.sqrt(2.0 / np.pi)
_TANH_A = 0.044715


def gelu(z, form: str = "erf"):
    """g(z) = z * Phi(z) (exact GeLU).

    form "tanh": the tanh approximation of Hendrycks & Gimpel, "Gaussian Error
    Linear Units (GELUs)", section 2: Phi(z) is replaced by
    (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3))) / 2.  No workload uses it; it is
    here to check the kernels' variant behind the GeLU flag."""
    z = np.asarray(z, dtype=np.float64)
    if form == "tanh":
        return 0.5 * z * (1.0 + np.tanh(_TANH_C * (z + _TANH_A * z ** 3)))
    if form != "erf":
        raise ValueError(form)
    return z * normal_cdf(z)


def gelu_grad(z, form: str = "erf"):
    """g'(z) = Phi(z) + z * phi(z); for the tanh form, with u = sqrt(2/pi) (z + 0.044715 z^3),
    d/dz [z (1 + tanh u) / 2] = (1 + tanh u) / 2 + z (1 - tanh^2 u) u'(z) / 2."""
    z = np.asarray(z, dtype=np.float64)
    if form == "tanh":
        t = np.tanh(_TANH_C * (z + _TANH_A * z ** 3))
        du = _TANH_C * (1.0 + 3.0 * _TANH_A * z * z)
        return 0.5 * (1.0 + t) + 0.5 * z * (1.0 - t * t) * du
    if form != "erf":
        raise ValueError(form)
    return normal_cdf(z) + z * normal_pdf(z)


# ------------------------------------------------------------------- linears
# [TUT] zero-bubble section; [ZB] section 3, B/W decomposition.

def linear_forward(x, w):
    """F of a linear: Y = X.W  (X [T,K], W [K,N])."""
    return x @ w


def linear_backward_input(dy, w):
    """B of a linear: dX = dY.W^T."""
    return dy @ w.T


def linear_backward_weight(x, dy):
    """W of a linear: dW = X^T.dY."""
    return x.T @ dy


# ----------------------------------------------------------------- attention

def causal_attention_forward(q, k, v):
    """One head, one sequence.  q, k, v: [s, d].  Returns O [s,d], P [s,s], LSE [s]."""
    s, d = q.shape
    scores = (q @ k.T) / np.sqrt(d)
    future = np.triu(np.ones((s, s), dtype=bool), k=1)
    scores = np.where(future, -np.inf, scores)
    row_max = scores.max(axis=1, keepdims=True)
    e = np.exp(scores - row_max)
    denom = e.sum(axis=1, keepdims=True)
    p = e / denom
    o = p @ v
    lse = (row_max + np.log(denom))[:, 0]
    return o, p, lse


def causal_attention_backward(q, k, v, p, do):
    """Gradients of one head from the saved probabilities P and dO."""
    d = q.shape[1]
    dv = p.T @ do
    dp = do @ v.T
    ds = p * (dp - (dp * p).sum(axis=1, keepdims=True))
    dq = (ds @ k) / np.sqrt(d)
    dk = (ds.T @ q) / np.sqrt(d)
    return dq, dk, dv


def _heads(h: int, n_heads: int):
    d = h // n_heads
    return [(i * d, (i + 1) * d) for i in range(n_heads)]


def multihead_forward(qkv, h, n_heads, seq):
    """qkv [T, 3h] (Q | K | V column blocks, head-major inside each); T = b*seq rows."""
    t = qkv.shape[0]
    o = np.zeros((t, h))
    lse = np.zeros((n_heads, t))
    probs = {}
    for b0 in range(0, t, seq):
        rows = slice(b0, b0 + seq)
        for hi, (c0, c1) in enumerate(_heads(h, n_heads)):
            q = qkv[rows, c0:c1]
            k = qkv[rows, h + c0:h + c1]
            v = qkv[rows, 2 * h + c0:2 * h + c1]
            oh, ph, lh = causal_attention_forward(q, k, v)
            o[rows, c0:c1] = oh
            lse[hi, rows] = lh
            probs[(b0, hi)] = ph
    return o, lse, probs


def multihead_backward(qkv, probs, do, h, n_heads, seq):
    t = qkv.shape[0]
    dqkv = np.zeros((t, 3 * h))
    for b0 in range(0, t, seq):
        rows = slice(b0, b0 + seq)
        for hi, (c0, c1) in enumerate(_heads(h, n_heads)):
            q = qkv[rows, c0:c1]
            k = qkv[rows, h + c0:h + c1]
            v = qkv[rows, 2 * h + c0:2 * h + c1]
            dq, dk, dv = causal_attention_backward(q, k, v, probs[(b0, hi)], do[rows, c0:c1])
            dqkv[rows, c0:c1] = dq
            dqkv[rows, h + c0:h + c1] = dk
            dqkv[rows, 2 * h + c0:2 * h + c1] = dv
    return dqkv


# --------------------------------------------------------------------- layer

def layer_forward(wl: si.Workload, W: Dict[str, np.ndarray], x: np.ndarray):
    """F of one layer.  Returns (y, saved) where saved holds what B and W need."""
    h = wl.hidden
    if wl.kind == si.TINY_MLP:
        z = linear_forward(x, W["up"])
        a = gelu(z, wl.gelu)
        y = linear_forward(a, W["down"])
        return y, {"x_up": x, "z": z, "a": a}
    if wl.kind == si.MLP_LINEARS:
        qkv = linear_forward(x, W["qkv"])
        o = qkv[:, 2 * h:3 * h].copy()
        p = linear_forward(o, W["proj"])
        z = linear_forward(p, W["up"])
        a = gelu(z, wl.gelu)
        y = linear_forward(a, W["down"])
        return y, {"x": x, "o": o, "x_up": p, "z": z, "a": a}
    qkv = linear_forward(x, W["qkv"])
    o, lse, probs = multihead_forward(qkv, h, wl.n_heads, wl.seq)
    x1 = x + linear_forward(o, W["proj"])
    z = linear_forward(x1, W["up"])
    a = gelu(z, wl.gelu)
    y = x1 + linear_forward(a, W["down"])
    return y, {"x": x, "qkv": qkv, "o": o, "lse": lse, "probs": probs,
               "x_up": x1, "z": z, "a": a}


def layer_backward_input(wl: si.Workload, W, saved, dy):
    """B of one layer: the input gradient dx, plus the output gradient of every
    linear (what its W pass consumes).  No weight gradient is formed here."""
    h = wl.hidden
    dz = linear_backward_input(dy, W["down"]) * gelu_grad(saved["z"], wl.gelu)
    if wl.kind == si.TINY_MLP:
        dx = linear_backward_input(dz, W["up"])
        return dx, {"up": dz, "down": dy}
    if wl.kind == si.MLP_LINEARS:
        dp = linear_backward_input(dz, W["up"])
        do = linear_backward_input(dp, W["proj"])
        dqkv = np.zeros((dy.shape[0], 3 * h))
        dqkv[:, 2 * h:3 * h] = do
        dx = linear_backward_input(dqkv, W["qkv"])
        return dx, {"qkv": dqkv, "proj": dp, "up": dz, "down": dy}
    dx1 = dy + linear_backward_input(dz, W["up"])
    do = linear_backward_input(dx1, W["proj"])
    dqkv = multihead_backward(saved["qkv"], saved["probs"], do, h, wl.n_heads, wl.seq)
    dx = dx1 + linear_backward_input(dqkv, W["qkv"])
    return dx, {"qkv": dqkv, "proj": dx1, "up": dz, "down": dy}


def linear_inputs(wl: si.Workload, saved) -> Dict[str, np.ndarray]:
    """The input X of every linear of the layer (what its W pass consumes)."""
    if wl.kind == si.TINY_MLP:
        return {"up": saved["x_up"], "down": saved["a"]}
    return {"qkv": saved["x"], "proj": saved["o"], "up": saved["x_up"], "down": saved["a"]}


def layer_backward_weight(wl: si.Workload, saved, grads) -> Dict[str, np.ndarray]:
    """W of one layer: dW = X^T.dY for every linear."""
    xs = linear_inputs(wl, saved)
    return {nm: linear_backward_weight(xs[nm], grads[nm]) for nm in grads}


def layer_backward_fused(wl: si.Workload, W, saved, dy):
    """Unsplit backward of one layer: walking the linears from the output back
    to the input, each linear yields its weight gradient and its input gradient
    in the same step (the conventional monolithic backward, [ZB] section 2)."""
    h = wl.hidden
    xs = linear_inputs(wl, saved)
    dws = {}
    dws["down"] = xs["down"].T @ dy
    dz = (dy @ W["down"].T) * gelu_grad(saved["z"], wl.gelu)
    dws["up"] = xs["up"].T @ dz
    if wl.kind == si.TINY_MLP:
        return dz @ W["up"].T, dws
    if wl.kind == si.MLP_LINEARS:
        dp = dz @ W["up"].T
        dws["proj"] = xs["proj"].T @ dp
        do = dp @ W["proj"].T
        dqkv = np.zeros((dy.shape[0], 3 * h))
        dqkv[:, 2 * h:] = do
        dws["qkv"] = xs["qkv"].T @ dqkv
        return dqkv @ W["qkv"].T, dws
    dx1 = dy + dz @ W["up"].T
    dws["proj"] = xs["proj"].T @ dx1
    do = dx1 @ W["proj"].T
    dqkv = multihead_backward(saved["qkv"], saved["probs"], do, h, wl.n_heads, wl.seq)
    dws["qkv"] = xs["qkv"].T @ dqkv
    return dx1 + dqkv @ W["qkv"].T, dws


# --------------------------------------------------------------------- stage

def to64(weights: Sequence[Dict[str, np.ndarray]]) -> List[Dict[str, np.ndarray]]:
    return [{k: np.asarray(v, dtype=np.float64) for k, v in l.items()} for l in weights]


def stage_forward(wl, weights, x):
    """F of a stage: its layers in order.  Returns (y, per-layer saved)."""
    saved = []
    for W in weights:
        x, s = layer_forward(wl, W, x)
        saved.append(s)
    return x, saved


def stage_backward_input(wl, weights, saved, dy):
    """B of a stage: layers in reverse.  Returns (dx, per-layer linear output grads)."""
    grads = [None] * len(weights)
    for li in range(len(weights) - 1, -1, -1):
        dy, grads[li] = layer_backward_input(wl, weights[li], saved[li], dy)
    return dy, grads


def stage_backward_weight(wl, saved, grads):
    """W of a stage for one microbatch: per-layer dict of dW."""
    return [layer_backward_weight(wl, s, g) for s, g in zip(saved, grads)]


def stage_backward_fused(wl, weights, saved, dy):
    dws = [None] * len(weights)
    for li in range(len(weights) - 1, -1, -1):
        dy, dws[li] = layer_backward_fused(wl, weights[li], saved[li], dy)
    return dy, dws


def add_grads(acc, dws):
    if acc is None:
        return [{k: v.copy() for k, v in l.items()} for l in dws]
    for a, d in zip(acc, dws):
        for k in a:
            a[k] += d[k]
    return acc


def pipeline(wl: si.Workload, weights_per_stage, xs, dys, w_order=None):
    """All P stages for all m microbatches, in fp64.

    Stage s output of microbatch j is stage s+1's input; the gradient that stage
    s+1's B returns is stage s's upstream gradient ([ZB] section 3, dependency
    rules).  ``xs[j]`` is the first stage's input, ``dys[j]`` the gradient
    entering the last stage.  ``w_order[s]`` is the order in which stage s adds
    its per-microbatch weight gradients (ascending by default).

    Returns dict with y[s][j], dx[s][j], dw[s] (summed over microbatches).
    """
    P, m = wl.n_stages, wl.n_micro
    ws = [to64(w) for w in weights_per_stage]
    y = [[None] * m for _ in range(P)]
    x_in = [[None] * m for _ in range(P)]
    saved = [[None] * m for _ in range(P)]
    for j in range(m):
        x = np.asarray(xs[j], dtype=np.float64)
        for s in range(P):
            x_in[s][j] = x
            x, saved[s][j] = stage_forward(wl, ws[s], x)
            y[s][j] = x
    dx = [[None] * m for _ in range(P)]
    grads = [[None] * m for _ in range(P)]
    for j in range(m):
        g = np.asarray(dys[j], dtype=np.float64)
        for s in range(P - 1, -1, -1):
            g, grads[s][j] = stage_backward_input(wl, ws[s], saved[s][j], g)
            dx[s][j] = g
    dw = []
    for s in range(P):
        order = list(range(m)) if w_order is None else list(w_order[s])
        acc = None
        for j in order:
            acc = add_grads(acc, stage_backward_weight(wl, saved[s][j], grads[s][j]))
        dw.append(acc)
    return {"x_in": x_in, "y": y, "dx": dx, "dw": dw, "saved": saved, "grads": grads}


def concat_microbatches(arrs):
    return np.concatenate([np.asarray(a, dtype=np.float64) for a in arrs], axis=0)


def stage_full_batch_fused(wl: si.Workload, weights, xs, dys):
    """Fused backward over the whole batch: all microbatches' tokens stacked
    into one pass (sequences stay separate inside attention).  Returns (y, dx, dw)."""
    ws = to64(weights)
    x = concat_microbatches(xs)
    dy = concat_microbatches(dys)
    y, saved = stage_forward(wl, ws, x)
    dx, dw = stage_backward_fused(wl, ws, saved, dy)
    return y, dx, dw
