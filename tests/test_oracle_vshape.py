"""Pins of the ZB-V oracle (oracle/vshape.py): the V placement, validity of its
orders, balanced per-device memory, its bubble against the handcrafted orders,
and the result of "Zero Bubble Pipeline Parallelism" section 6 at equal pass
times: zero bubble with P M_B per device.  An exhaustive search on the smallest
pipeline (written here, independent of the oracle's own search) shows such an
order exists; the built orders reach it for P = 2 .. 8.
"""
import json
import os
import random

import pytest

from oracle import schedules as S
from oracle import vshape as V

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
UNIT = {"F": 1, "B": 1, "W": 1}


@pytest.mark.parametrize("P", [1, 2, 3, 8])
def test_placement_is_a_v(P):
    # device d holds chunks d and 2P-1-d; a microbatch's forward visits the
    # devices 0..P-1 and back, so the first device also runs the last chunk
    assert [V.device_of(c, P) for c in range(2 * P)] == list(range(P)) + list(range(P - 1, -1, -1))
    for d in range(P):
        assert sorted(c for c in range(2 * P) if V.device_of(c, P) == d) == [d, 2 * P - 1 - d]


def _check(P, m, orders, t, m_b, m_w, m_limit, t_comm=0):
    sim = V.simulate(P, orders, t, t_comm)
    lin = V.linearize(orders, sim)
    assert S.validate_linear(2 * P, m, lin) == (S.OK, -1)
    for d, o in enumerate(orders):
        assert len(o) == 6 * m
        assert all(V.device_of(c, P) == d for _, c, _ in o)
        assert V.peak_memory(o, m_b, m_w) <= m_limit
        for c in (d, 2 * P - 1 - d):
            ws = [j for k, cc, j in o if k == "W" and cc == c]
            assert ws == list(range(m))
    return sim


@pytest.mark.parametrize("seed", range(6))
def test_orders_valid_and_within_budget(seed):
    rng = random.Random(seed)
    for _ in range(50):
        P, m = rng.randint(1, 6), rng.randint(1, 12)
        t = {"F": rng.randint(1, 5), "B": rng.randint(1, 6), "W": rng.randint(1, 4)}
        m_b, m_w = rng.randint(1, 5), rng.randint(1, 5)
        m_limit = max(m_w, rng.randint(2 * m_b + max(0, m_w - m_b), 3 * P * m_b + m_w))
        comm = rng.choice([0, 0, 1, 3])
        orders = V.build(P, m, t, m_b, m_w, m_limit, comm)
        sim = _check(P, m, orders, t, m_b, m_w, m_limit, comm)
        assert sim.makespan >= sim.ideal


def test_budget_below_one_microbatch_is_rejected():
    with pytest.raises(ValueError):
        V.build(4, 8, UNIT, 2, 3, 4)   # needs 2 M_B + (M_W - M_B) = 5


@pytest.mark.parametrize("P", [2, 4])
def test_memory_is_balanced_at_p_mb(P):
    """Every device peaks at the same level, P M_B of a whole stage (2P chunk
    stashes), where ZB-H2's first stage holds (2P-1) whole-stage M_B."""
    for m in (2 * P, 3 * P):
        orders = V.build(P, m, UNIT, 1, 1, 2 * P)
        _check(P, m, orders, UNIT, 1, 1, 2 * P)
        assert [V.peak_memory(o, 1, 1) for o in orders] == [2 * P] * P
        h2 = S.stage_orders("zbh2", P, m)
        assert S.peak_memory(h2[0], 2, 2) == 2 * (2 * P - 1)   # in chunk units: a stage's M_B = 2


def _rate(sim):
    return sim.bubble / sim.makespan


def test_profiled_times_beat_zbh1_and_1f1b():
    """At the pages' profiled pass times (Table 9; a chunk takes half a stage's
    time), the V order's bubble rate is below ZB-H1's and 1F1B's, with half of
    ZB-H2's memory (section 6's comparison, Table 8)."""
    g = json.load(open(os.path.join(GOLDEN, "zb_table9_profiled_times.json")))
    for row in g["rows"]:
        t = {k: int(round(1000 * row["T_" + k])) for k in "FBW"}
        half = {k: v // 2 for k, v in t.items()}
        for P, m in ((8, row["m"]), (16, 48)):
            sim = _check(P, m, V.build(P, m, half, 1, 1, 2 * P), half, 1, 1, 2 * P)
            f1, h1 = (S.simulate(S.stage_orders(n, P, m), {k: 2 * v for k, v in half.items()}) for n in ("1f1b", "zbh1"))
            assert _rate(sim) < _rate(h1) < _rate(f1)


@pytest.mark.parametrize("P,m", [(2, 4), (4, 8), (8, 24)])
def test_equal_times_list_candidate_below_zbh1(P, m):
    sim = V.simulate(P, V.list_orders(P, m, UNIT, 1, 1, 2 * P), UNIT)
    h1 = S.simulate(S.stage_orders("zbh1", P, m), {"F": 2, "B": 2, "W": 2})
    assert 0 <= sim.bubble < h1.bubble


def _zero_bubble_at_p_mb(P, m, t, m_b, m_w):
    limit = 2 * P * m_b
    orders = V.build(P, m, t, m_b, m_w, limit)
    sim = _check(P, m, orders, t, m_b, m_w, limit)
    assert sim.bubble == 0 and sim.makespan == sim.ideal
    assert all(c == sim.ideal for c in sim.device_cost)
    assert [V.peak_memory(o, m_b, m_w) for o in orders] == [limit] * P


@pytest.mark.parametrize("P,m", [(2, 4), (2, 8), (3, 6), (4, 8), (4, 12), (5, 10), (6, 12)])
@pytest.mark.parametrize("m_b,m_w", [(1, 1), (3, 2)])
def test_equal_times_zero_bubble_within_p_mb(P, m, m_b, m_w):
    """Section 6's result: at T_F = T_B = T_W the V order has no bubble (every
    device busy from its first pass to its last) and every device peaks at
    exactly P M_B of a whole stage, 2P chunk stashes; the same holds when a W
    stash is smaller than a B stash (the pages' M_W < M_B)."""
    for t in (UNIT, {"F": 5, "B": 5, "W": 5}):
        _zero_bubble_at_p_mb(P, m, t, m_b, m_w)


def test_equal_times_zero_bubble_eight_devices():
    _zero_bubble_at_p_mb(8, 16, UNIT, 1, 1)


@pytest.mark.parametrize("P,m", [(4, 32), (8, 24)])
def test_search_scales_with_microbatches(P, m):
    orders = V.search_order(P, m, 1, 1, 2 * P)
    assert orders is not None
    sim = _check(P, m, orders, UNIT, 1, 1, 2 * P)
    assert sim.bubble == 0


def test_search_gives_up_below_the_warm_up():
    """With fewer than 2P - 1 microbatches a device cannot fill its warm-up with
    forwards; the search reports no order and build keeps the list order."""
    assert V.search_order(4, 6, 1, 1, 8) is None
    assert V.search_order(4, 7, 1, 1, 8) is not None
    orders = V.build(4, 6, UNIT, 1, 1, 8)
    assert orders == V.list_orders(4, 6, UNIT, 1, 1, 8)
    assert V.simulate(4, orders, UNIT).bubble > 0


def test_unequal_times_keep_the_list_order():
    t = {"F": 3, "B": 4, "W": 2}
    assert V.build(4, 8, t, 1, 1, 8) == V.list_orders(4, 8, t, 1, 1, 8)


def _zero_bubble_v_exists(P, m, cap):
    """Depth-first search over every V order at unit pass times in which no
    device idles between its first and last pass, with at most `cap` chunk
    stashes live per device (F +1, W -1)."""
    C = 2 * P
    nf, nb = [0] * C, [0] * C
    end_f, end_b = {}, {}
    wq = [[] for _ in range(P)]
    mem, done, started = [0] * P, [0] * P, [False] * P

    def moves(d, t):
        out = []
        for c in (2 * P - 1 - d, d):
            j = nb[c]
            if j < nf[c] and end_f[(c, j)] <= t and (c == C - 1 or end_b.get((c + 1, j), t + 1) <= t):
                out.append(("B", c))
        for c in (2 * P - 1 - d, d):
            j = nf[c]
            if j < m and mem[d] < cap and (c == 0 or end_f.get((c - 1, j), t + 1) <= t):
                out.append(("F", c))
        if wq[d]:
            out.append(("W", None))
        return out

    def step(t):
        if all(x == 6 * m for x in done):
            return True
        choices = []
        for d in range(P):
            if done[d] == 6 * m:
                choices.append([None])
                continue
            mv = moves(d, t)
            if not mv:
                if started[d]:
                    return False
                choices.append([None])
            else:
                choices.append(mv)

        def assign(d):
            if d == P:
                return step(t + 1)
            for mv in choices[d]:
                if mv is None:
                    if assign(d + 1):
                        return True
                    continue
                k, c = mv
                if k == "F":
                    j = nf[c]; nf[c] += 1; end_f[(c, j)] = t + 1; mem[d] += 1
                elif k == "B":
                    j = nb[c]; nb[c] += 1; end_b[(c, j)] = t + 1; wq[d].append((c, j))
                else:
                    c, j = wq[d].pop(0); mem[d] -= 1
                was = started[d]; started[d] = True; done[d] += 1
                if assign(d + 1):
                    return True
                done[d] -= 1; started[d] = was
                if k == "F":
                    nf[c] -= 1; del end_f[(c, j)]; mem[d] -= 1
                elif k == "B":
                    nb[c] -= 1; del end_b[(c, j)]; wq[d].pop()
                else:
                    wq[d].insert(0, (c, j)); mem[d] += 1
            return False
        return assign(0)

    return step(0)


def test_zero_bubble_v_order_exists_within_p_mb():
    """The pages' claim at equal pass times, checked by exhaustive search on the
    smallest V (P = 2, m = 4): an order with no idle time inside any device's
    span exists within 2P chunk stashes (P M_B), and none within one stash
    less.  The built order reaches it; the list-scheduled candidate alone is
    one chunk pass above it."""
    assert _zero_bubble_v_exists(2, 4, 4)
    assert not _zero_bubble_v_exists(2, 4, 3)
    assert V.search_order(2, 4, 1, 1, 3) is None
    assert V.simulate(2, V.build(2, 4, UNIT, 1, 1, 4), UNIT).bubble == 0
    assert V.simulate(2, V.list_orders(2, 4, UNIT, 1, 1, 4), UNIT).bubble == 1
