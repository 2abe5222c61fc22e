"""Planned-versus-observed join of an executed schedule (measurement only).

"Zero-Bubble Pipeline Parallelism, Proven", section "Validate the schedule as
data": keep the plan as the control and the runtime trace as the result, join
them by event id, report start and duration errors, and separate time spent
waiting for a producer (dependency wait) from time spent waiting for a busy
executor (resource wait).

Here an event id is the pass (stage, kind, microbatch).  The executor runs
the passes of the emulated stages on a few HIP streams of one GPU; a stream
is the exclusive resource of the passes issued to it, in list order.  The
plan places every pass as soon as its stream is free and its producers have
ended (the dependency rules of the executor: F(s-1,j) before F(s,j), F(s,j)
before B(s,j), B(s+1,j) before B(s,j), B(s,j) before W(s,j), with U standing
for B), using planned durations per (stage, kind).  From a timeline (planned
or observed) the waits of a pass are, with `free` the end of the previous pass
on its stream and `ready` the latest end of its producers:
  dependency wait = max(0, min(start, ready) - free) (the stream idled until a
                    producer on another stream ended);
  resource wait   = max(0, min(start, free) - ready) (the pass was ready but
                    its stream was still busy with other passes).
No arithmetic of the method is done here.
"""
from __future__ import annotations

from typing import Dict, List, Sequence, Tuple

Op = Tuple[int, str, int]


def producers(op: Op, P: int) -> List[Op]:
    """Passes that must end before `op` starts (cross-stage and same-stage)."""
    s, k, j = op
    if k == "F":
        return [(s - 1, "F", j)] if s > 0 else []
    if k in ("B", "U"):
        deps = [(s, "F", j)]
        if s + 1 < P:
            deps += [(s + 1, "B", j), (s + 1, "U", j)]
        return deps
    if k == "W":
        return [(s, "B", j)]
    return []


def plan_timeline(ops: Sequence[Op], P: int, stream_of_stage: Sequence[int],
                  durations: Dict[Tuple[int, str], float]) -> Dict[Op, Tuple[float, float]]:
    """ASAP placement of `ops` (the executor's list order) on the streams."""
    free: Dict[int, float] = {}
    end: Dict[Op, float] = {}
    out: Dict[Op, Tuple[float, float]] = {}
    for op in ops:
        st = stream_of_stage[op[0]]
        ready = max([end[d] for d in producers(op, P) if d in end], default=0.0)
        t0 = max(free.get(st, 0.0), ready)
        t1 = t0 + durations[(op[0], op[1])]
        out[op] = (t0, t1)
        end[op] = t1
        free[st] = t1
    return out


def waits(ops: Sequence[Op], P: int, stream_of_stage: Sequence[int],
          timeline: Dict[Op, Tuple[float, float]]) -> Dict[Op, Tuple[float, float]]:
    """(dependency wait, resource wait) of every pass of a timeline."""
    free: Dict[int, float] = {}
    out = {}
    for op in ops:
        st = stream_of_stage[op[0]]
        t0, t1 = timeline[op]
        ready = max([timeline[d][1] for d in producers(op, P) if d in timeline], default=0.0)
        f = free.get(st, 0.0)
        dep = max(0.0, min(t0, ready) - f)
        res = max(0.0, min(t0, f) - ready)
        out[op] = (dep, res)
        free[st] = t1
    return out


def _summary(xs: List[float]) -> Dict[str, float]:
    if not xs:
        return {"median": 0.0, "p90": 0.0, "max_abs": 0.0}
    ys = sorted(xs)
    return {"median": ys[len(ys) // 2], "p90": ys[min(len(ys) - 1, (9 * len(ys)) // 10)],
            "max_abs": max(abs(v) for v in ys)}


def median_durations(trace) -> Dict[Tuple[int, str], float]:
    """Median traced duration (ms) of each (stage, kind)."""
    by: Dict[Tuple[int, str], List[float]] = {}
    for (op, ms, _) in trace:
        by.setdefault((op[0], op[1]), []).append(ms)
    return {k: sorted(v)[len(v) // 2] for k, v in by.items()}


def join(ops: Sequence[Op], P: int, stream_of_stage: Sequence[int], trace,
         durations: Dict[Tuple[int, str], float], top: int = 5) -> dict:
    """Joins a traced run (records (op, ms, t0_ms) in list order) with its plan
    built from `durations` (ms per (stage, kind)).  Returns errors and waits in
    milliseconds."""
    obs = {op: (t0, t0 + ms) for (op, ms, t0) in trace}
    plan = plan_timeline(ops, P, stream_of_stage, durations)
    w_obs = waits(ops, P, stream_of_stage, obs)
    w_plan = waits(ops, P, stream_of_stage, plan)
    start_err = {op: obs[op][0] - plan[op][0] for op in ops}
    dur_err = {op: (obs[op][1] - obs[op][0]) - (plan[op][1] - plan[op][0]) for op in ops}
    worst = sorted(ops, key=lambda o: -abs(dur_err[o]))[:top]
    return {
        "passes": len(ops),
        "streams": len(set(stream_of_stage)),
        "planned_span_ms": max(t1 for (_, t1) in plan.values()),
        "observed_span_ms": max(t1 for (_, t1) in obs.values()),
        "start_error_ms": _summary(list(start_err.values())),
        "duration_error_ms": _summary(list(dur_err.values())),
        "dependency_wait_ms": {"planned": sum(d for d, _ in w_plan.values()),
                               "observed": sum(d for d, _ in w_obs.values())},
        "resource_wait_ms": {"planned": sum(r for _, r in w_plan.values()),
                             "observed": sum(r for _, r in w_obs.values())},
        "largest_duration_errors": [{"op": f"{k}({s},{j})", "planned_ms": plan[(s, k, j)][1] - plan[(s, k, j)][0],
                                     "observed_ms": obs[(s, k, j)][1] - obs[(s, k, j)][0]}
                                    for (s, k, j) in worst],
    }
