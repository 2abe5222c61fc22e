"""Oracle of the automatic (heuristic) zero-bubble scheduler, ZB-1p / ZB-2p.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Plain Python, integer
times and memory; no code is shared with the native schedule layer.

Follows the four phases that "Zero Bubble Pipeline Parallelism" gives for its
heuristic (section 3.1, as the structured summary describes them under "The
Heuristic Scheduling Algorithm"): warm-up forwards while the activation memory
stays within M_limit, a steady state that alternates F and B and fills gaps
with W, a forward-count balance between neighbouring stages, and a cool-down
that drains the remaining W; two binary choices are searched and the order
with the smallest makespan kept.  Where the pages leave a step open, this is
the plain reading (stated again in the design notes):

* The schedule is built by list scheduling in time: the stage that becomes
  free first (ties: lower stage) picks its next pass among those whose
  producers are already placed.
* The stage's "next primary pass" is F while it is warming up (no B placed
  yet), then B and F alternate, B first; F stops being primary once all m
  forwards are placed, B once all m backwards are.
* Memory is charged at the start of a pass, as in the memory ledger: F adds
  M_B, B adds M_W - M_B, W adds -M_W; a forward also keeps room for its own B
  (max(0, M_W - M_B)).  A primary F that would exceed M_limit yields to a
  pending W (the memory-triggered W), else to B; a B that would exceed it
  yields to W; else the stage waits.
* fill (first binary choice): during warm-up, a forward that would end after
  the first B could start is still placed (fill = 1) or the stage switches to
  B (fill = 0).
* balance (second binary choice): the pages' invariant that a stage has
  placed at least one forward more than the next stage, applied while the
  stage warms up.  With balance = 1 a warm-up forward on stage s > 0 is
  skipped unless stage s-1 will still be ahead after it (or has placed all m
  forwards); the stage's first forward is never skipped, so that a budget
  that holds few microbatches cannot leave a stage with nothing to run.
* Gap filling: when the primary pass is not ready, a pending W (ascending
  microbatch) fills the gap if the gap is at least T_W, or if leaving the gap
  idle would make this stage's accumulated idle time the largest of all
  stages; otherwise the stage waits.
* Cool-down: with every F and B placed, the remaining W run in ascending order.
* The result is scored with the ordinary simulator (Eq. 3 stage cost); the
  four (fill, balance) combinations are tried in the order (0,0), (0,1),
  (1,0), (1,1) and the first with the smallest makespan is kept.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Tuple

from .schedules import Op, simulate

INF = float("inf")


def build(P: int, m: int, t: Dict[str, int], m_b: int, m_w: int, m_limit: int, fill: int, balance: int,
          t_comm: int = 0) -> List[List[Op]]:
    """Per-stage pass orders for one (fill, balance) choice."""
    if P < 1 or m < 1:
        raise ValueError("P and m must be >= 1")
    if m_b < 0 or m_w < 0 or m_limit < max(m_b, m_w):
        raise ValueError("M_limit below one microbatch in flight")
    delta = {"F": m_b, "B": m_w - m_b, "W": -m_w}
    reserve = max(0, m_w - m_b)      # a forward leaves room for its own B
    orders: List[List[Op]] = [[] for _ in range(P)]
    n_f = [0] * P
    n_b = [0] * P
    w_q: List[List[int]] = [[] for _ in range(P)]
    mem = [0] * P
    free = [0] * P
    idle = [0] * P                   # idle time after the stage's first pass
    last: List[Optional[str]] = [None] * P  # last F or B placed (a W does not break the alternation)
    end_f: Dict[Tuple[int, int], int] = {}
    end_b: Dict[Tuple[int, int], int] = {}
    total = 3 * P * m
    placed = 0

    def active(s: int) -> bool:
        return len(orders[s]) < 3 * m

    def ready_f(s: int) -> float:
        if s == 0:
            return 0
        e = end_f.get((s - 1, n_f[s]))
        return INF if e is None else e + t_comm

    def ready_b(s: int) -> float:
        j = n_b[s]
        r = end_f.get((s, j))
        if r is None:
            return INF
        if s < P - 1:
            e = end_b.get((s + 1, j))
            if e is None:
                return INF
            r = max(r, e + t_comm)
        return r

    def primary(s: int) -> Optional[str]:
        f_left, b_ready_mb = n_f[s] < m, n_b[s] < n_f[s]
        if n_b[s] == 0:                          # warm-up
            return "F" if f_left else ("B" if b_ready_mb else None)
        if not f_left:
            return "B" if n_b[s] < m else None
        if last[s] == "B" or not b_ready_mb:     # steady state: F after B
            return "F"
        return "B"

    def place(s: int, kind: str, now: int) -> None:
        nonlocal placed
        if kind == "F":
            j = n_f[s]
            start = max(now, ready_f(s))
            n_f[s] += 1
            end_f[(s, j)] = start + t["F"]
        elif kind == "B":
            j = n_b[s]
            start = max(now, ready_b(s))
            n_b[s] += 1
            end_b[(s, j)] = start + t["B"]
            w_q[s].append(j)
        else:
            j = w_q[s].pop(0)
            start = now
        if orders[s]:
            idle[s] += start - now
        mem[s] += delta[kind]
        free[s] = start + t[kind]
        orders[s].append((kind, j))
        if kind != "W":
            last[s] = kind
        placed += 1

    def decide(s: int, now: int):
        """('place', kind) | ('wait', time) | ('defer', None): the next step of stage s at `now`."""
        p = primary(s)
        if p == "F":
            full = mem[s] + delta["F"] + reserve > m_limit
            if full and w_q[s]:
                return ("place", "W")            # memory-triggered W: free a microbatch's stash first
            blocked = full
            if balance and n_b[s] == 0 and 0 < n_f[s] and s > 0 and n_f[s - 1] < m and n_f[s - 1] < n_f[s] + 2:
                blocked = True                   # warm-up: keep one forward of lead on the upstream stage
            if blocked:
                p = "B" if n_b[s] < n_f[s] else None
            elif n_b[s] == 0 and n_b[s] < n_f[s] and not fill:
                rb = ready_b(s)
                if rb < INF and max(now, ready_f(s)) + t["F"] > rb:
                    p = "B"                      # one more forward would delay the first B
        if p == "B" and mem[s] + delta["B"] > m_limit:
            p = None
        r = ready_f(s) if p == "F" else (ready_b(s) if p == "B" else INF)
        if p is not None and r <= now:
            return ("place", p)
        if w_q[s]:
            gap = r - now
            if p is None or gap >= t["W"] or (orders[s] and idle[s] + gap > max(idle)):
                return ("place", "W")
        if p is not None and r < INF:
            return ("wait", r)
        return ("defer", None)

    while placed < total:
        now = min(free[s] for s in range(P) if active(s))
        progress = True
        while progress:                          # stages at `now` re-decide while others place passes
            progress = False
            for s in range(P):
                if not active(s) or free[s] != now:
                    continue
                what, arg = decide(s, now)
                if what == "place":
                    place(s, arg, now)
                    progress = True
                elif what == "wait":
                    if orders[s]:
                        idle[s] += arg - now
                    free[s] = arg
        later = [free[q] for q in range(P) if active(q) and free[q] > now]
        stuck = [s for s in range(P) if active(s) and free[s] == now]
        if stuck:
            if not later:
                raise RuntimeError("heuristic: no stage can progress")
            nxt = min(later)
            for s in stuck:
                if orders[s]:
                    idle[s] += nxt - now
                free[s] = nxt
    return orders


def schedule(P: int, m: int, t: Dict[str, int], m_b: int, m_w: int, m_limit: int,
             t_comm: int = 0) -> Tuple[List[List[Op]], int, int, int]:
    """The grid search: returns (orders, makespan, fill, balance) of the best combination."""
    best = None
    for fill in (0, 1):
        for balance in (0, 1):
            orders = build(P, m, t, m_b, m_w, m_limit, fill, balance, t_comm)
            ms = simulate(orders, t, t_comm).makespan
            if best is None or ms < best[1]:
                best = (orders, ms, fill, balance)
    return best
