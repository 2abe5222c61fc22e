"""Oracle of the pipeline schedules: pass orders, simulator, accounting, validators.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Plain Python on small
integers; no code is shared with the native schedule layer.

Pass kinds: 'F' forward, 'B' input gradient, 'W' weight gradient, and 'U' an
unsplit backward (B and W run as one pass, the conventional backward).

Dependencies ([ZB] section 3, "The Backward Pass Decomposition", and its ILP
appendix, Eq. 4-5): F(s,j) after F(s-1,j); B(s,j) after F(s,j) and after the
backward of (s+1,j); W(s,j) after B(s,j) only.  The optimizer of a step needs
every W of that step ([AUD] "Draw the event graph before the Gantt").

Stages are 0-indexed here: stage s of P.  The pages count from 1.
"""
from __future__ import annotations

from dataclasses import dataclass
from fractions import Fraction
from typing import Dict, List, Sequence, Tuple

Op = Tuple[str, int]  # (kind, microbatch) on one stage


# ------------------------------------------------------------ pass orders

def order_gpipe(P: int, m: int, s: int) -> List[Op]:
    """GPipe: every forward, then every (unsplit) backward ([TUT] "The problem GPipe leaves behind")."""
    return [("F", j) for j in range(m)] + [("U", j) for j in range(m)]


def order_1f1b(P: int, m: int, s: int) -> List[Op]:
    """1F1B ([TUT] "1F1B: same bubble, bounded memory"): stage s first runs
    P-1-s warm-up forwards, then alternates one forward with one unsplit
    backward, then drains the remaining backwards."""
    warm = min(m, P - 1 - s)
    ops = [("F", j) for j in range(warm)]
    next_f = warm
    for b in range(m):
        if next_f < m:
            ops.append(("F", next_f))
            next_f += 1
        ops.append(("U", b))
    return ops


def order_zbh1(P: int, m: int, s: int) -> List[Op]:
    """ZB-H1 ([ZB] "Handcrafted Schedule ZB-H1"): the forwards and B passes sit
    where 1F1B puts its forwards and backwards; the W passes are delayed.  Stage
    s holds back s weight-gradient passes, so its peak is (P-s) M_B + s M_W,
    the same M_B count as 1F1B, and the held-back W's fill the drain."""
    warm = min(m, P - 1 - s)
    ops = [("F", j) for j in range(warm)]
    next_f, next_w = warm, 0
    for b in range(m):
        if next_f < m:
            ops.append(("F", next_f))
            next_f += 1
        ops.append(("B", b))
        if b >= s:
            ops.append(("W", next_w))
            next_w += 1
    ops += [("W", j) for j in range(next_w, m)]
    return ops


def order_zbh2(P: int, m: int, s: int) -> List[Op]:
    """ZB-H2 ([ZB] "Handcrafted Schedule ZB-H2"): stage s runs 2(P-s)-1
    forwards before its first B (2P-1 on the first stage, as in the paper's
    P=4, m=8 example with seven forwards), then repeats B, W, F with the W's
    held back by 2s passes so that the tail forms a parallelogram."""
    warm = min(m, 2 * (P - s) - 1)
    ops = [("F", j) for j in range(warm)]
    next_f, next_w = warm, 0
    for b in range(m):
        ops.append(("B", b))
        if b >= 2 * s:
            ops.append(("W", next_w))
            next_w += 1
        if next_f < m:
            ops.append(("F", next_f))
            next_f += 1
    ops += [("W", j) for j in range(next_w, m)]
    return ops


def order_w_last(P: int, m: int, s: int) -> List[Op]:
    """ZB-H1's forward/B placement with every W deferred after the stage's last B
    (the latest legal place before the optimizer)."""
    ops = [op for op in order_zbh1(P, m, s) if op[0] != "W"]
    return ops + [("W", j) for j in range(m)]


ORDERS = {"gpipe": order_gpipe, "1f1b": order_1f1b, "zbh1": order_zbh1,
          "zbh2": order_zbh2, "wlast": order_w_last}


def stage_orders(name: str, P: int, m: int) -> List[List[Op]]:
    return [ORDERS[name](P, m, s) for s in range(P)]


# -------------------------------------------------------------- simulator

@dataclass
class SimResult:
    start: Dict[Tuple[int, str, int], int]    # (stage, kind, mb) -> start time
    end: Dict[Tuple[int, str, int], int]
    stage_cost: List[int]                     # Eq. 3: last end - first start
    makespan: int                             # max over stages of stage_cost
    span: int                                 # max end over all passes (all start at t >= 0)
    busy: int                                 # total pass time
    ideal: int                                # m (T_F + T_B + T_W)

    @property
    def bubble(self) -> int:
        """[ZB] section 5 "Metrics": cost - m(T_F+T_B+T_W), cost = largest stage time."""
        return self.makespan - self.ideal

    @property
    def bubble_rate(self) -> Fraction:
        return Fraction(self.bubble, self.makespan)

    def global_ratio(self, P: int) -> Fraction:
        """[AUD] checker's ratio: 1 - busy / (stages * span)."""
        return 1 - Fraction(self.busy, P * self.span)


def _duration(kind: str, t: Dict[str, int]) -> int:
    return t["B"] + t["W"] if kind == "U" else t[kind]


def simulate(orders: Sequence[Sequence[Op]], t: Dict[str, int], t_comm: int = 0) -> SimResult:
    """As-soon-as-possible execution of fixed per-stage orders.

    A pass starts at the later of: its stage becoming free, and each producer's
    end (+ t_comm when the producer sits on a neighbouring stage), following
    [ZB] ILP appendix Eq. 4-6.  Raises RuntimeError on a deadlock.
    """
    P = len(orders)
    start: Dict[Tuple[int, str, int], int] = {}
    end: Dict[Tuple[int, str, int], int] = {}
    back_end: Dict[Tuple[int, int], int] = {}  # (stage, mb) -> end of its B or U
    pos = [0] * P
    free = [0] * P
    remaining = sum(len(o) for o in orders)
    while remaining:
        progressed = False
        for s in range(P):
            while pos[s] < len(orders[s]):
                kind, j = orders[s][pos[s]]
                ready = free[s]
                deps_ok = True
                if kind == "F":
                    if s > 0:
                        if (s - 1, "F", j) not in end:
                            deps_ok = False
                        else:
                            ready = max(ready, end[(s - 1, "F", j)] + t_comm)
                elif kind in ("B", "U"):
                    if (s, "F", j) not in end:
                        deps_ok = False
                    else:
                        ready = max(ready, end[(s, "F", j)])
                    if deps_ok and s < P - 1:
                        if (s + 1, j) not in back_end:
                            deps_ok = False
                        else:
                            ready = max(ready, back_end[(s + 1, j)] + t_comm)
                elif kind == "W":
                    if (s, "B", j) not in end:
                        deps_ok = False
                    else:
                        ready = max(ready, end[(s, "B", j)])
                else:
                    raise ValueError(kind)
                if not deps_ok:
                    break
                dur = _duration(kind, t)
                start[(s, kind, j)] = ready
                end[(s, kind, j)] = ready + dur
                if kind in ("B", "U"):
                    back_end[(s, j)] = ready + dur
                free[s] = ready + dur
                pos[s] += 1
                remaining -= 1
                progressed = True
        if not progressed:
            raise RuntimeError("deadlock: no stage can start its next pass")
    costs = []
    for s in range(P):
        first = orders[s][0]
        last = orders[s][-1]
        costs.append(end[(s, last[0], last[1])] - start[(s, first[0], first[1])])
    m = max(j for o in orders for _, j in o) + 1
    busy = sum(_duration(k, t) for o in orders for k, _ in o)
    return SimResult(start, end, costs, max(costs), max(end.values()), busy,
                     m * (t["F"] + t["B"] + t["W"]))


def linearize(orders: Sequence[Sequence[Op]], sim: SimResult) -> List[Tuple[int, str, int]]:
    """One-device execution order: by simulated start time, ties to the lower stage."""
    items = [(sim.start[(s, k, j)], s, idx, k, j)
             for s, o in enumerate(orders) for idx, (k, j) in enumerate(o)]
    items.sort(key=lambda r: (r[0], r[1], r[2]))
    return [(s, k, j) for _, s, _, k, j in items]


# ------------------------------------------- interleaved (virtual stages)

def simulate_interleaved(P: int, m: int, v: int, t_chunk: Dict[str, int]) -> SimResult:
    """Interleaved pipeline ([TUT] "Interleaved stages"): device d holds model
    chunks c = 0..v-1, i.e. virtual stages k = c*P + d.  Forwards go group by
    group of P microbatches, chunk 0 to v-1; backwards (unsplit) go group by
    group, chunk v-1 down to 0.  Per-chunk times are ``t_chunk``.
    Dependencies run along the virtual stages."""
    if m % P:
        raise ValueError("interleaved order needs m divisible by P")
    V = v * P
    groups = [list(range(g, g + P)) for g in range(0, m, P)]
    dev_orders = []
    for d in range(P):
        o = []
        for g in groups:
            for c in range(v):
                o += [("F", c * P + d, j) for j in g]
        for g in groups:
            for c in range(v - 1, -1, -1):
                o += [("U", c * P + d, j) for j in g]
        dev_orders.append(o)
    start, end = {}, {}
    pos = [0] * P
    free = [0] * P
    remaining = sum(len(o) for o in dev_orders)
    while remaining:
        progressed = False
        for d in range(P):
            while pos[d] < len(dev_orders[d]):
                kind, k, j = dev_orders[d][pos[d]]
                ready = free[d]
                if kind == "F":
                    dep = (k - 1, "F", j) if k > 0 else None
                else:
                    dep = (k + 1, "U", j) if k < V - 1 else (k, "F", j)
                if dep is not None and dep not in end:
                    break
                if dep is not None:
                    ready = max(ready, end[dep])
                if kind == "U" and (k, "F", j) in end:
                    ready = max(ready, end[(k, "F", j)])
                dur = _duration(kind, t_chunk)
                start[(k, kind, j)] = ready
                end[(k, kind, j)] = ready + dur
                free[d] = ready + dur
                pos[d] += 1
                remaining -= 1
                progressed = True
        if not progressed:
            raise RuntimeError("deadlock")
    costs = []
    for d in range(P):
        f = dev_orders[d][0]
        l = dev_orders[d][-1]
        costs.append(end[(l[1], l[0], l[2])] - start[(f[1], f[0], f[2])])
    busy = sum(_duration(kd, t_chunk) for o in dev_orders for kd, _, _ in o)
    ideal = m * v * (t_chunk["F"] + t_chunk["B"] + t_chunk["W"])
    return SimResult(start, end, costs, max(costs), max(end.values()), busy, ideal)


# ---------------------------------------------------------- memory ledger

def memory_profile(order: Sequence[Op], m_b, m_w) -> List:
    """Running activation memory of one stage ([ZB] "The Memory Model"):
    F adds M_B, B adds M_W - M_B, W adds -M_W; an unsplit backward adds -M_B.
    Each increment is charged at the start of its pass (ILP appendix Eq. 7).
    Returns the level after each pass."""
    delta = {"F": m_b, "B": m_w - m_b, "W": -m_w, "U": -m_b}
    level, out = 0, []
    for k, _ in order:
        level += delta[k]
        out.append(level)
    return out


def peak_memory(order: Sequence[Op], m_b, m_w):
    return max([0] + memory_profile(order, m_b, m_w))


# --------------------------------------------------- order validator (untimed)

OK, E_ARG, E_DUPLICATE, E_INVALID_STAGE, E_INVALID_MB, E_MISSING, E_DEPENDENCY = (
    "ok", "arg", "duplicate", "invalid_stage", "invalid_mb", "missing", "dependency")


def validate_linear(P: int, m: int, ops: Sequence[Tuple[int, str, int]]) -> Tuple[str, int]:
    """Check a one-device execution order of (stage, kind, mb) passes.

    Rules, checked pass by pass in list order, first failure wins:
      kind in {F,B,W,U}                                  else 'arg'
      0 <= stage < P                                     else 'invalid_stage'
      0 <= mb < m                                        else 'invalid_mb'
      no pass repeated; B/U and W/U exclusive            else 'duplicate'
      F(s,j) after F(s-1,j); B|U(s,j) after F(s,j) and
      after B|U(s+1,j); W(s,j) after B(s,j)              else 'dependency'
    then completeness: every (s,j) has F and either B and W, or U; else
    'missing' at index len(ops).  ([ZB] section 3 dependency rules; [AUD]
    "Validate the schedule as data" error classes; the optimizer dependency of
    [AUD] "Draw the event graph" is the completeness rule.)
    Returns (status, index of the first failing pass, or -1).
    """
    done = set()   # (stage, kind, mb)
    for i, (s, k, j) in enumerate(ops):
        if k not in ("F", "B", "W", "U"):
            return E_ARG, i
        if not (0 <= s < P):
            return E_INVALID_STAGE, i
        if not (0 <= j < m):
            return E_INVALID_MB, i
        if (s, k, j) in done:
            return E_DUPLICATE, i
        if k == "U" and ((s, "B", j) in done or (s, "W", j) in done):
            return E_DUPLICATE, i
        if k in ("B", "W") and (s, "U", j) in done:
            return E_DUPLICATE, i
        if k == "F":
            if s > 0 and (s - 1, "F", j) not in done:
                return E_DEPENDENCY, i
        elif k in ("B", "U"):
            if (s, "F", j) not in done:
                return E_DEPENDENCY, i
            if s < P - 1 and (s + 1, "B", j) not in done and (s + 1, "U", j) not in done:
                return E_DEPENDENCY, i
        else:  # W
            if (s, "B", j) not in done:
                return E_DEPENDENCY, i
        done.add((s, k, j))
    for s in range(P):
        for j in range(m):
            has_f = (s, "F", j) in done
            split = (s, "B", j) in done and (s, "W", j) in done
            if not has_f or not (split or (s, "U", j) in done):
                return E_MISSING, len(ops)
    return OK, -1


# ------------------------------------------------ timed event inspector

class ScheduleError(Exception):
    pass


def _interval_ok(t) -> bool:
    return t["start"] >= 0 and t["end"] > t["start"]


def inspect_events(tasks: Sequence[dict], stage_count) -> dict:
    """Checks a schedule given as timed events, following the prose of [AUD]
    "Validate the schedule as data" (reject duplicate ids, unknown stages,
    invalid intervals, missing dependencies, consumers that begin before their
    producers end, and overlapping work on one stage; report span, busy time,
    the idle ratio under a stated denominator and the activations still held)
    and "Budget activation lifetime" (an activation is held from its F to the
    W that consumes the stash its B leaves).

    Each task: id, stage, micro, kind, start, end, optional depends_on.
    Checks run in phases; within a phase the reported task is fixed as stated:
      1. stage_count < 1                          -> invalid_stage_count
      2. an id seen before                        -> duplicate_task (its second use)
      3. stage outside [0, stage_count)           -> invalid_stage  (first in list order)
      4. start < 0 or end <= start                -> invalid_interval (first in list order)
      5. a dependency id that names no task       -> missing_dependency (first in list order)
      6. a task starting before a producer ends   -> dependency_violation: the violating
                                                     task with the earliest start, ties to
                                                     the list order
      7. two tasks of one stage overlapping       -> stage_overlap: of every overlapping
                                                     pair the later-starting task (ties: later
                                                     in the list); the smallest (start, index)
    Report: span = latest end (time starts at 0), busy = sum of durations,
    bubble_ratio = 1 - busy / (stage_count * span), unfinished_activations =
    (stage, micro) activations whose F has run but whose stash no W (or
    unsplit U) has released, peak_live_activations = the most held at once by
    one stage.  Written as plain brute force over all tasks and pairs.
    """
    if not isinstance(stage_count, int) or isinstance(stage_count, bool) or stage_count < 1:
        raise ScheduleError("invalid_stage_count")
    n = len(tasks)
    for i in range(n):
        for k in range(i):
            if tasks[k]["id"] == tasks[i]["id"]:
                raise ScheduleError("duplicate_task", i)
    for i, t in enumerate(tasks):
        st = t["stage"]
        if not isinstance(st, int) or isinstance(st, bool) or not 0 <= st < stage_count:
            raise ScheduleError("invalid_stage", i)
    for i, t in enumerate(tasks):
        if not _interval_ok(t):
            raise ScheduleError("invalid_interval", i)
    ids = [t["id"] for t in tasks]
    for i, t in enumerate(tasks):
        for d in t.get("depends_on", []):
            if d not in ids:
                raise ScheduleError("missing_dependency", i)
    violators = []
    for i, t in enumerate(tasks):
        producers = [tasks[ids.index(d)] for d in t.get("depends_on", [])]
        if any(p["end"] > t["start"] for p in producers):
            violators.append((t["start"], i))
    if violators:
        raise ScheduleError("dependency_violation", min(violators)[1])
    overlaps = []
    for i in range(n):
        for k in range(n):
            a, b = tasks[i], tasks[k]
            if i == k or a["stage"] != b["stage"]:
                continue
            later = (b["start"], k) > (a["start"], i)
            if later and a["start"] < b["end"] and b["start"] < a["end"]:
                overlaps.append((b["start"], k))
    if overlaps:
        raise ScheduleError("stage_overlap", min(overlaps)[1])
    span = max(t["end"] for t in tasks)
    busy = sum(t["end"] - t["start"] for t in tasks)
    # Activation ledger: walk the tasks by start time (ties in list order).
    held = {}
    peak = 0
    for _, i in sorted((t["start"], i) for i, t in enumerate(tasks)):
        t = tasks[i]
        key = (t["stage"], t["micro"])
        if t["kind"] == "F":
            held[key] = held.get(key, 0) + 1
        elif t["kind"] in ("W", "U"):
            held[key] = max(0, held.get(key, 0) - 1)
        peak = max(peak, sum(v for (s, _), v in held.items() if s == t["stage"]))
    return {"span": span, "busy": busy,
            "bubble_ratio": 1 - Fraction(busy) / (stage_count * Fraction(span)),
            "unfinished_activations": sum(held.values()),
            "peak_live_activations": peak}
