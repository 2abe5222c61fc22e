"""Oracle of the optimizer step with post-update validation and in-place AdamW rollback.

TEST INFRASTRUCTURE ONLY (see the package docstring).  numpy fp64; no code is
shared with the device path.

"Zero Bubble Pipeline Parallelism", section 4 ("The Optimizer Synchronization
Bypass" in the structured summary) and its Appendix C (Algorithm 1, described
there in words and by the AdamW update formula):

* each stage's local state after the step boundary is the sum of its squared
  gradients and whether any gradient is NaN/Inf;
* staged reduce: stage s combines its local state with the partial state of
  stage s-1 and hands the result on; the last stage holds the global state;
* optimistic step: each stage steps at once with the partial state it has:
  gradients clipped when the partial norm exceeds the threshold, no update
  when a NaN/Inf has been seen;
* validation: the global state travels back from the last stage; a stage
  whose step differs from the one the global state calls for rolls it back by
  inverting AdamW exactly (given the same gradient) and steps again with the
  global state.

Readings (stated again in the design notes): the clip coefficient is
min(1, max_norm / (norm + 1e-6)) of the usual gradient-norm clipping; a step
"differs" when its clip coefficient differs or its skip decision differs; the
AdamW update is the one the page prints (decoupled weight decay applied to
the pre-step parameters, bias-corrected moments, epsilon outside the root).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional, Sequence, Tuple

import numpy as np

State = Tuple[float, bool]   # (sum of squared gradients, any NaN/Inf)


@dataclass(frozen=True)
class AdamW:
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.01
    max_grad_norm: float = 1.0     # <= 0: no clipping


def local_state(grads: Sequence[np.ndarray]) -> State:
    """One stage's contribution: sum of squares of its gradients, non-finite flag."""
    sumsq = 0.0
    bad = False
    for g in grads:
        g64 = np.asarray(g, dtype=np.float64)
        bad |= not bool(np.all(np.isfinite(g64)))
        sumsq += float(np.sum(g64 * g64))
    return sumsq, bad


def combine(upstream: Optional[State], local: State) -> State:
    """Staged reduce step: partial state of stage s from that of s-1 and its own."""
    if upstream is None:
        return local
    return upstream[0] + local[0], upstream[1] or local[1]


def staged_reduce(locals_: Sequence[State]) -> List[State]:
    """Partial states of stages 0..P-1; the last one is the global state."""
    out: List[State] = []
    for st in locals_:
        out.append(combine(out[-1] if out else None, st))
    return out


def clip_coef(state: State, hp: AdamW) -> Optional[float]:
    """Gradient multiplier for a step taken with `state`; None = skip the update."""
    sumsq, bad = state
    if bad or not np.isfinite(sumsq):
        return None
    if hp.max_grad_norm <= 0:
        return 1.0
    return min(1.0, hp.max_grad_norm / (float(np.sqrt(sumsq)) + 1e-6))


def adamw_step(theta, m, v, grad, coef: Optional[float], step: int, hp: AdamW):
    """AdamW step number `step` (1-based) with gradient coef * grad; returns the
    new (theta, m, v).  No change when coef is None (skipped step)."""
    theta, m, v = (np.asarray(x, dtype=np.float64) for x in (theta, m, v))
    if coef is None:
        return theta.copy(), m.copy(), v.copy()
    g = coef * np.asarray(grad, dtype=np.float64)
    m1 = hp.beta1 * m + (1.0 - hp.beta1) * g
    v1 = hp.beta2 * v + (1.0 - hp.beta2) * g * g
    mhat = m1 / (1.0 - hp.beta1 ** step)
    vhat = v1 / (1.0 - hp.beta2 ** step)
    theta1 = theta - hp.lr * hp.weight_decay * theta - hp.lr * mhat / (np.sqrt(vhat) + hp.eps)
    return theta1, m1, v1


def adamw_rollback(theta1, m1, v1, grad, coef: Optional[float], step: int, hp: AdamW):
    """Inverse of adamw_step given the same gradient and coefficient: the
    update term is rebuilt from the post-step moments, then the moments are
    unwound (Appendix C's in-place rollback)."""
    theta1, m1, v1 = (np.asarray(x, dtype=np.float64) for x in (theta1, m1, v1))
    if coef is None:
        return theta1.copy(), m1.copy(), v1.copy()
    g = coef * np.asarray(grad, dtype=np.float64)
    mhat = m1 / (1.0 - hp.beta1 ** step)
    vhat = v1 / (1.0 - hp.beta2 ** step)
    theta = (theta1 + hp.lr * mhat / (np.sqrt(vhat) + hp.eps)) / (1.0 - hp.lr * hp.weight_decay)
    m = (m1 - (1.0 - hp.beta1) * g) / hp.beta1
    v = (v1 - (1.0 - hp.beta2) * g * g) / hp.beta2
    return theta, m, v


def needs_rollback(used: State, glob: State, hp: AdamW) -> bool:
    return clip_coef(used, hp) != clip_coef(glob, hp)


def validate(theta1, m1, v1, grad, used: State, glob: State, step: int, hp: AdamW):
    """Post-update validation of one tensor: (theta, m, v, rolled_back)."""
    if not needs_rollback(used, glob, hp):
        return (np.asarray(theta1, dtype=np.float64).copy(), np.asarray(m1, dtype=np.float64).copy(),
                np.asarray(v1, dtype=np.float64).copy(), False)
    theta, m, v = adamw_rollback(theta1, m1, v1, grad, clip_coef(used, hp), step, hp)
    theta, m, v = adamw_step(theta, m, v, grad, clip_coef(glob, hp), step, hp)
    return theta, m, v, True


def post_validated_step(params, moms, vels, grads, step: int, hp: AdamW):
    """The whole protocol over P stages (lists per stage of lists of tensors):
    staged reduce, optimistic steps with the partial states, validation with
    the global state.  Returns (params, moms, vels, rolled_back per stage)."""
    P = len(params)
    partial = staged_reduce([local_state(grads[s]) for s in range(P)])
    glob = partial[-1]
    out_p, out_m, out_v, rolled = [], [], [], []
    for s in range(P):
        coef = clip_coef(partial[s], hp)
        ps, ms, vs = [], [], []
        r_any = False
        for th, m, v, g in zip(params[s], moms[s], vels[s], grads[s]):
            th1, m1, v1 = adamw_step(th, m, v, g, coef, step, hp)
            th2, m2, v2, r = validate(th1, m1, v1, g, partial[s], glob, step, hp)
            ps.append(th2)
            ms.append(m2)
            vs.append(v2)
            r_any |= r
        out_p.append(ps)
        out_m.append(ms)
        out_v.append(vs)
        rolled.append(r_any)
    return out_p, out_m, out_v, rolled


def synchronous_step(params, moms, vels, grads, step: int, hp: AdamW):
    """The conventional step the protocol must reproduce: one global state
    before any stage updates."""
    P = len(params)
    glob = staged_reduce([local_state(grads[s]) for s in range(P)])[-1]
    coef = clip_coef(glob, hp)
    res = [[adamw_step(th, m, v, g, coef, step, hp) for th, m, v, g in zip(params[s], moms[s], vels[s], grads[s])]
           for s in range(P)]
    return ([[r[0] for r in rs] for rs in res], [[r[1] for r in rs] for rs in res],
            [[r[2] for r in rs] for rs in res])
