"""Oracle of the V-shaped placement and its schedule, ZB-V.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Plain Python on small
integers; no code is shared with the native schedule layer.

"Zero Bubble Pipeline Parallelism", section 6 (the structured summary's
"The V-Shaped Interleaving Pattern" and the ZB-V results): the model is cut
into 2P chunks and device d (0-indexed) holds chunks d and 2P-1-d, so a
microbatch's forward runs down the devices and back up, and its backward runs
the same path in reverse.  The pages give the placement and the properties
(activation memory P M_B per device, balanced across devices; bubbles close to
ZB-H2's) but not the order of passes.  The plain reading built here (stated
again in the design notes):

* Chunks are virtual stages 0..2P-1 of one chain: F(c,j) after F(c-1,j);
  B(c,j) after F(c,j) and B(c+1,j); W(c,j) after B(c,j).  A hand-off between
  chunks on different devices costs t_comm, on the same device nothing.
* Pass times are per chunk (half a stage's layers).  Memory per chunk pass:
  F +M_B, B +(M_W - M_B), W -M_W, charged at the start, with M_B, M_W those of
  one chunk.
* The order is built by list scheduling in time: the device that is free
  first (ties: lower device) takes, among its candidate passes, the one that
  can start earliest, ties broken in the order B of the earlier chunk, F of
  the later chunk, F of the earlier chunk, B of the later chunk; the oldest
  pending W (ascending per chunk) runs when nothing else can start at once.
* Memory: a forward of the earlier chunk also keeps room for the later
  chunk's forward of a microbatch and for a B's growth (2 M_B + max(0, M_W -
  M_B) over the current level), a forward of the later chunk room for its own
  B; a pass over M_limit is not a candidate, and a stage over the budget with
  a W pending runs that W.  M_limit for ZB-V is P M_B of a whole stage = 2P
  chunk M_B.
* At equal pass times the section's result is zero bubble within P M_B.  The
  list-scheduled order does not reach it, so a second candidate is searched
  (search_order): passes are unit slots, device d works in every slot from d
  to d + 6m - 1, and a depth-first search fills the slots device by device.
  Of the two candidates the one with the smaller simulated makespan at the
  given times is kept (ties: the searched one).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, List, Optional, Sequence, Tuple

VOp = Tuple[str, int, int]  # (kind, chunk, microbatch) on one device


def device_of(c: int, P: int) -> int:
    """Device holding chunk c: chunks d and 2P-1-d share device d ([ZB] section 6)."""
    return c if c < P else 2 * P - 1 - c


SEARCH_BUDGET = 1_000_000   # search steps before the searched candidate is given up


def build(P: int, m: int, t: Dict[str, int], m_b: int, m_w: int, m_limit: int,
          t_comm: int = 0) -> List[List[VOp]]:
    """Per-device pass orders of the V schedule: the list-scheduled order, or at
    equal pass times the searched zero-bubble order when it is not slower."""
    if P < 1 or m < 1:
        raise ValueError("P and m must be >= 1")
    reserve = max(0, m_w - m_b)
    if m_b < 0 or m_w < 0 or m_limit < 2 * m_b + reserve or m_limit < m_w:
        raise ValueError("M_limit below one microbatch through both chunks")
    listed = list_orders(P, m, t, m_b, m_w, m_limit, t_comm)
    if not t["F"] == t["B"] == t["W"]:
        return listed
    found = search_order(P, m, m_b, m_w, m_limit)
    if found is None:
        return listed
    if simulate(P, found, t, t_comm).makespan <= simulate(P, listed, t, t_comm).makespan:
        return found
    return listed


def list_orders(P: int, m: int, t: Dict[str, int], m_b: int, m_w: int, m_limit: int,
                t_comm: int = 0) -> List[List[VOp]]:
    """The list-scheduled candidate (rules in the module docstring)."""
    reserve = max(0, m_w - m_b)
    C = 2 * P
    nf = [0] * C
    nb = [0] * C
    end_f: Dict[Tuple[int, int], int] = {}
    end_b: Dict[Tuple[int, int], int] = {}
    w_q: List[List[Tuple[int, int]]] = [[] for _ in range(P)]
    mem = [0] * P
    free = [0] * P
    orders: List[List[VOp]] = [[] for _ in range(P)]

    def hop(c_from: int, c_to: int) -> int:
        return 0 if device_of(c_from, P) == device_of(c_to, P) else t_comm

    def ready_f(c: int) -> Optional[int]:
        j = nf[c]
        if j >= m:
            return None
        if c == 0:
            return 0
        e = end_f.get((c - 1, j))
        return None if e is None else e + hop(c - 1, c)

    def ready_b(c: int) -> Optional[int]:
        j = nb[c]
        if j >= nf[c]:
            return None
        r = end_f[(c, j)]
        if c < C - 1:
            e = end_b.get((c + 1, j))
            if e is None:
                return None
            r = max(r, e + hop(c + 1, c))
        return r

    def candidates(d: int):
        lo, hi = d, C - 1 - d
        now = free[d]
        out = []   # (start, rank, kind, chunk)
        r = ready_b(lo)
        if r is not None and mem[d] + m_w - m_b <= m_limit:
            out.append((max(now, r), 0, "B", lo))
        r = ready_f(hi)
        if r is not None and mem[d] + m_b + reserve <= m_limit:
            out.append((max(now, r), 1, "F", hi))
        r = ready_f(lo)
        if r is not None and mem[d] + 2 * m_b + reserve <= m_limit:
            out.append((max(now, r), 2, "F", lo))
        r = ready_b(hi)
        if r is not None and mem[d] + m_w - m_b <= m_limit:
            out.append((max(now, r), 3, "B", hi))
        if w_q[d]:
            full = not out or mem[d] + m_b + reserve > m_limit
            start = min(x[0] for x in out) if out else None
            if full or start > now:
                out.append((now, 4, "W", w_q[d][0][0]))
        return out

    total = 6 * P * m
    placed = 0
    while placed < total:
        best = None
        for d in range(P):
            if len(orders[d]) == 6 * m:
                continue
            for st, rank, kind, c in candidates(d):
                key = (st, d, rank)
                if best is None or key < best[0]:
                    best = (key, d, kind, c)
        if best is None:
            raise RuntimeError("zb-v: no device can progress")
        (st, _, _), d, kind, c = best
        if kind == "F":
            j = nf[c]
            nf[c] += 1
            end_f[(c, j)] = st + t["F"]
            mem[d] += m_b
        elif kind == "B":
            j = nb[c]
            nb[c] += 1
            end_b[(c, j)] = st + t["B"]
            w_q[d].append((c, j))
            mem[d] += m_w - m_b
        else:
            c, j = w_q[d].pop(0)
            mem[d] -= m_w
        orders[d].append((kind, c, j))
        free[d] = st + t[kind]
        placed += 1
    return orders


def latest_starts(P: int, m: int) -> Dict[Tuple[str, int, int], int]:
    """Latest slot of every chunk pass when device d works in slots d .. d+6m-1.

    A pass must leave room for everything that depends on it: each successor
    starts at least one slot later (F(c+1,j) and B(c,j) after F(c,j); B(c-1,j)
    and W(c,j) after B(c,j); the same pass of microbatch j+1 after j), and no
    pass ends after its device's last slot."""
    C = 2 * P
    L: Dict[Tuple[str, int, int], int] = {}
    for j in range(m - 1, -1, -1):
        for c in range(C):
            cap = device_of(c, P) + 6 * m - 1
            if j + 1 < m:
                cap = min(cap, L[("W", c, j + 1)] - 1)
            L[("W", c, j)] = cap
        for c in range(C):
            cap = min(device_of(c, P) + 6 * m - 1, L[("W", c, j)] - 1)
            if c > 0:
                cap = min(cap, L[("B", c - 1, j)] - 1)
            if j + 1 < m:
                cap = min(cap, L[("B", c, j + 1)] - 1)
            L[("B", c, j)] = cap
        for c in range(C - 1, -1, -1):
            cap = min(device_of(c, P) + 6 * m - 1, L[("B", c, j)] - 1)
            if c + 1 < C:
                cap = min(cap, L[("F", c + 1, j)] - 1)
            if j + 1 < m:
                cap = min(cap, L[("F", c, j + 1)] - 1)
            L[("F", c, j)] = cap
    return L


def search_order(P: int, m: int, m_b: int, m_w: int, m_limit: int,
                 budget: int = SEARCH_BUDGET) -> Optional[List[List[VOp]]]:
    """A V order with no idle slot inside any device's span at unit pass times,
    within m_limit per device, or None (none found within the budget).

    Slots are filled in time order, device 0 to P-1 within a slot; a device
    picks among the passes whose producers finished before the slot began.
    Choices are tried by urgency: the pass's latest start (latest_starts; for
    microbatches more than P+1 before the last, the value of microbatch m-P-1
    less six slots per microbatch, so that early microbatches are as urgent as
    in a short pipeline), then W before F before B, then the earlier chunk.
    After each slot the branch is cut when a pending pass is past its latest
    start, or when some device cannot have work in every coming slot even if
    all other devices ran every chain as early as it allows."""
    C = 2 * P
    lst = latest_starts(P, m)
    h = P + 1

    def urgency(k: str, c: int, j: int) -> int:
        if m > h and j < m - h:
            return lst[(k, c, m - h)] - 6 * (m - h - j)
        return lst[(k, c, j)]

    cnt = {"F": [0] * C, "B": [0] * C, "W": [0] * C}
    done = [0] * P
    orders: List[List[VOp]] = [[] for _ in range(P)]
    rank = {"W": 0, "F": 1, "B": 2}

    # Stashes live per device (forward started, W not yet): at most `room`, so
    # that the ledger level, at most max(M_B, M_W) per live stash, stays
    # within m_limit whatever the ratio of M_B to M_W.
    room = m_limit // max(m_b, m_w) if max(m_b, m_w) > 0 else 2 * m

    def choices(d: int, snap) -> List[Tuple[str, int]]:
        sF, sB, sW = snap
        live = sum(sF[c] - sW[c] for c in (d, C - 1 - d))
        out = []
        for c in (d, C - 1 - d):
            if sF[c] < m and live < room and (c == 0 or sF[c - 1] > sF[c]):
                out.append(("F", c))
            if sB[c] < sF[c] and (c == C - 1 or sB[c + 1] > sB[c]):
                out.append(("B", c))
            if sW[c] < sB[c]:
                out.append(("W", c))
        out.sort(key=lambda kc: (urgency(kc[0], kc[1], cnt[kc[0]][kc[1]]), rank[kc[0]]))
        return out

    def hopeless(t: int) -> bool:
        for k in "FBW":
            for c in range(C):
                j = cnt[k][c]
                if j < m and lst[(k, c, j)] < t:
                    return True
        est: Dict[Tuple[str, int, int], int] = {}
        for j in range(m):
            for c in range(C):
                if cnt["F"][c] <= j:
                    e = t
                    if c > 0 and ("F", c - 1, j) in est:
                        e = max(e, est[("F", c - 1, j)] + 1)
                    if j > 0 and ("F", c, j - 1) in est:
                        e = max(e, est[("F", c, j - 1)] + 1)
                    est[("F", c, j)] = e
            for c in range(C - 1, -1, -1):
                if cnt["B"][c] <= j:
                    e = t
                    if ("F", c, j) in est:
                        e = max(e, est[("F", c, j)] + 1)
                    if c < C - 1 and ("B", c + 1, j) in est:
                        e = max(e, est[("B", c + 1, j)] + 1)
                    if j > 0 and ("B", c, j - 1) in est:
                        e = max(e, est[("B", c, j - 1)] + 1)
                    est[("B", c, j)] = e
                if cnt["W"][c] <= j:
                    e = t
                    if ("B", c, j) in est:
                        e = max(e, est[("B", c, j)] + 1)
                    if j > 0 and ("W", c, j - 1) in est:
                        e = max(e, est[("W", c, j - 1)] + 1)
                    est[("W", c, j)] = e
        for d in range(P):
            if done[d] == 6 * m:
                continue
            mine = sorted(e for (k, c, j), e in est.items() if device_of(c, P) == d)
            first = max(t, d)
            if any(e > first + i for i, e in enumerate(mine)):
                return True
        return False

    # Depth-first search with an explicit stack.  A level is (slot t, device d);
    # d == P closes the slot.  Each level holds its choices and the index of the
    # one applied; None stands for a device that is finished or not started.
    snaps = {}
    stack = []
    steps = 0

    def enter(t: int, d: int) -> Optional[list]:
        nonlocal steps
        steps += 1
        if steps > budget:
            raise TimeoutError
        if d == P:
            if all(x == 6 * m for x in done):
                return ["done"]
            if hopeless(t + 1):
                return []
            snaps[t + 1] = (tuple(cnt["F"]), tuple(cnt["B"]), tuple(cnt["W"]))
            return [None]
        if done[d] == 6 * m or t < d:
            return [None]
        return choices(d, snaps[t])

    snaps[0] = (tuple(cnt["F"]), tuple(cnt["B"]), tuple(cnt["W"]))
    try:
        stack.append([0, 0, enter(0, 0), -1])
        while stack:
            top = stack[-1]
            t, d, opts, i = top
            if opts and opts[0] == "done":
                return orders
            if i >= 0 and opts[i] is not None:
                k, c = opts[i]
                cnt[k][c] -= 1
                done[d] -= 1
                orders[d].pop()
            i += 1
            top[3] = i
            if i >= len(opts):
                stack.pop()
                continue
            if opts[i] is not None:
                k, c = opts[i]
                orders[d].append((k, c, cnt[k][c]))
                cnt[k][c] += 1
                done[d] += 1
            nt, nd = (t + 1, 0) if d == P else (t, d + 1)
            stack.append([nt, nd, enter(nt, nd), -1])
    except TimeoutError:
        return None
    return None


@dataclass
class VSimResult:
    start: Dict[Tuple[int, str, int], int]   # (chunk, kind, mb) -> start
    end: Dict[Tuple[int, str, int], int]
    device_cost: List[int]                   # Eq. 3 per device: last end - first start
    makespan: int
    ideal: int                               # 2 m (T_F + T_B + T_W) in chunk pass times

    @property
    def bubble(self) -> int:
        return self.makespan - self.ideal


def simulate(P: int, orders: Sequence[Sequence[VOp]], t: Dict[str, int], t_comm: int = 0) -> VSimResult:
    """As-soon-as-possible execution of fixed per-device orders on the V chain."""
    C = 2 * P
    start: Dict[Tuple[int, str, int], int] = {}
    end: Dict[Tuple[int, str, int], int] = {}
    pos = [0] * P
    free = [0] * P
    remaining = sum(len(o) for o in orders)
    while remaining:
        progressed = False
        for d in range(P):
            while pos[d] < len(orders[d]):
                kind, c, j = orders[d][pos[d]]
                deps = []
                if kind == "F" and c > 0:
                    deps.append((c - 1, "F", j))
                elif kind == "B":
                    deps.append((c, "F", j))
                    if c < C - 1:
                        deps.append((c + 1, "B", j))
                elif kind == "W":
                    deps.append((c, "B", j))
                if any(x not in end for x in deps):
                    break
                r = free[d]
                for x in deps:
                    r = max(r, end[x] + (0 if device_of(x[0], P) == d else t_comm))
                start[(c, kind, j)] = r
                end[(c, kind, j)] = r + t[kind]
                free[d] = r + t[kind]
                pos[d] += 1
                remaining -= 1
                progressed = True
        if not progressed:
            raise RuntimeError("deadlock: no device can start its next pass")
    costs = []
    for d, o in enumerate(orders):
        (k0, c0, j0), (k1, c1, j1) = o[0], o[-1]
        costs.append(end[(c1, k1, j1)] - start[(c0, k0, j0)])
    m = max(j for o in orders for _, _, j in o) + 1
    return VSimResult(start, end, costs, max(costs), 2 * m * (t["F"] + t["B"] + t["W"]))


def linearize(orders: Sequence[Sequence[VOp]], sim: VSimResult) -> List[Tuple[int, str, int]]:
    """One-device order over the 2P chunk stages: by simulated start, ties to the lower chunk."""
    items = [(sim.start[(c, k, j)], c, idx, k, j)
             for o in orders for idx, (k, c, j) in enumerate(o)]
    items.sort(key=lambda r: (r[0], r[1], r[2]))
    return [(c, k, j) for _, c, _, k, j in items]


def peak_memory(order: Sequence[VOp], m_b: int, m_w: int) -> int:
    """Largest activation level of one device, charged at the start of each pass."""
    level = peak = 0
    for k, _, _ in order:
        level += {"F": m_b, "B": m_w - m_b, "W": -m_w}[k]
        peak = max(peak, level)
    return peak
