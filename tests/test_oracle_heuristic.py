"""Pins of the automatic-scheduler oracle (oracle/heuristic.py).

What the pages fix ("Zero Bubble Pipeline Parallelism", section 3.1 and the
memory model; section 5): every order respects the dependencies and the
activation-memory budget; with 1F1B's memory (M_limit = P M_B, ZB-1p) the
automatic schedule does better than 1F1B and as well as the handcrafted
ZB-H1; with twice that memory (ZB-2p) it reaches zero bubble at equal pass
times and is never worse than ZB-H2.  Independently of the pages' claims, a
brute-force search over every legal order of tiny pipelines bounds it from
below, and it reaches that optimum there.
"""
import itertools
import random

import pytest

from oracle import heuristic as H
from oracle import schedules as S

EQUAL = {"F": 1, "B": 1, "W": 1}
# Pass-time triples (T_F, T_B, T_W) with T_W the shortest, as the pages assume,
# plus the profiled ratio family of [ZB] Table 9 scaled to integers.
TIMES = [EQUAL, {"F": 2, "B": 3, "W": 1}, {"F": 18, "B": 18, "W": 10}, {"F": 3, "B": 4, "W": 2},
         {"F": 2, "B": 2, "W": 1}, {"F": 1, "B": 2, "W": 1}]


def _check_valid(P, m, orders, t, m_b, m_w, m_limit, t_comm=0):
    sim = S.simulate(orders, t, t_comm)
    lin = S.linearize(orders, sim)
    assert S.validate_linear(P, m, lin) == (S.OK, -1)
    for o in orders:
        assert S.peak_memory(o, m_b, m_w) <= m_limit
        ws = [j for k, j in o if k == "W"]
        assert ws == sorted(ws) and len(ws) == m
    return sim


@pytest.mark.parametrize("seed", range(6))
def test_orders_valid_and_within_budget(seed):
    rng = random.Random(seed)
    for _ in range(60):
        P, m = rng.randint(1, 6), rng.randint(1, 12)
        t = {"F": rng.randint(1, 5), "B": rng.randint(1, 6), "W": rng.randint(1, 4)}
        m_b, m_w = rng.randint(1, 5), rng.randint(1, 5)
        m_limit = rng.randint(max(m_b, m_w), (2 * P + 1) * m_b + m_w)
        comm = rng.choice([0, 0, 1, 3])
        orders, ms, _, _ = H.schedule(P, m, t, m_b, m_w, m_limit, comm)
        sim = _check_valid(P, m, orders, t, m_b, m_w, m_limit, comm)
        assert sim.makespan == ms >= sim.ideal


def test_budget_below_one_microbatch_is_rejected():
    with pytest.raises(ValueError):
        H.build(4, 8, EQUAL, 2, 3, 2, 0, 0)


@pytest.mark.parametrize("P", [2, 4, 8])
@pytest.mark.parametrize("t", TIMES)
def test_zb1p_beats_1f1b_and_matches_zbh1(P, t):
    m_b, m_w = 2, 1
    for m in (2 * P, 3 * P):
        orders, _, _, _ = H.schedule(P, m, t, m_b, m_w, P * m_b)
        sim = _check_valid(P, m, orders, t, m_b, m_w, P * m_b)
        f1 = S.simulate(S.stage_orders("1f1b", P, m), t)
        h1 = S.simulate(S.stage_orders("zbh1", P, m), t)
        assert sim.bubble < f1.bubble
        assert sim.bubble <= h1.bubble
        # the first stage holds no more than 1F1B's P microbatches
        assert S.peak_memory(orders[0], m_b, m_w) <= P * m_b


# Stash ledgers where B adds memory (M_W > M_B) or frees little (M_W close to
# M_B): with 1F1B's own peak as the budget (P microbatches' M_B plus the growth
# M_W - M_B of the one microbatch in its backward), the automatic order is never
# worse than 1F1B, for any pass times.
@pytest.mark.parametrize("m_b,m_w", [(34, 32), (28, 32), (22, 32), (1, 2)])
@pytest.mark.parametrize("P,m", [(2, 4), (4, 8), (4, 12), (8, 24)])
def test_zb1p_never_worse_than_1f1b_any_ledger(m_b, m_w, P, m):
    budget = P * m_b + max(0, m_w - m_b)
    for tf, tb, tw in itertools.product(range(1, 5), repeat=3):
        t = {"F": tf, "B": tb, "W": tw}
        orders, ms, _, _ = H.schedule(P, m, t, m_b, m_w, budget)
        for o in orders:
            assert S.peak_memory(o, m_b, m_w) <= budget
        assert ms <= S.simulate(S.stage_orders("1f1b", P, m), t).makespan, t


def _memory_triggered_w_holds(orders, m, m_b, m_w, budget):
    """Whenever a stage's next primary pass is F, the forward would pass the
    budget and a W is pending, the stage's next pass is that W."""
    reserve = max(0, m_w - m_b)
    for o in orders:
        mem, n_f, n_b, pending, last = 0, 0, 0, 0, None
        for k, _ in o:
            primary_f = n_f < m and (n_b == 0 or last == "B" or n_b == n_f)
            if primary_f and pending and mem + m_b + reserve > budget and k != "W":
                return False
            mem += {"F": m_b, "B": m_w - m_b, "W": -m_w}[k]
            n_f += k == "F"
            n_b += k == "B"
            pending += {"F": 0, "B": 1, "W": -1}[k]
            if k != "W":
                last = k
    return True


def test_memory_triggered_w():
    rng = random.Random(3)
    for _ in range(200):
        P, m = rng.randint(2, 6), rng.randint(2, 12)
        t = {"F": rng.randint(1, 4), "B": rng.randint(1, 4), "W": rng.randint(1, 4)}
        m_b, m_w = rng.randint(1, 4), rng.randint(1, 4)
        budget = rng.randint(max(m_b, m_w), 2 * P * m_b)
        for fill in (0, 1):
            for balance in (0, 1):
                orders = H.build(P, m, t, m_b, m_w, budget, fill, balance)
                assert _memory_triggered_w_holds(orders, m, m_b, m_w, budget)


@pytest.mark.parametrize("P", [2, 4, 8])
@pytest.mark.parametrize("t", TIMES)
def test_zb2p_never_worse_than_zbh2(P, t):
    m_b, m_w = 2, 1
    for m in (2 * P, 3 * P):
        orders, _, _, _ = H.schedule(P, m, t, m_b, m_w, 2 * P * m_b)
        sim = _check_valid(P, m, orders, t, m_b, m_w, 2 * P * m_b)
        h2 = S.simulate(S.stage_orders("zbh2", P, m), t)
        assert sim.bubble <= h2.bubble


@pytest.mark.parametrize("P", [2, 4, 8, 16])
def test_zb2p_zero_bubble_at_equal_times(P):
    for m in (2 * P - 1, 2 * P, 3 * P):
        orders, _, _, _ = H.schedule(P, m, EQUAL, 2, 1, 2 * P * 2)
        assert S.simulate(orders, EQUAL).bubble == 0


def _stage_sequences(m):
    """Every order of one stage's F (in order), B (in order) and W (ascending)
    passes with B_j after F_j and W_j after B_j."""
    out = []

    def rec(nf, nb, nw, seq):
        if nw == m:
            out.append(list(seq))
            return
        if nf < m:
            rec(nf + 1, nb, nw, seq + [("F", nf)])
        if nb < nf:
            rec(nf, nb + 1, nw, seq + [("B", nb)])
        if nw < nb:
            rec(nf, nb, nw + 1, seq + [("W", nw)])

    rec(0, 0, 0, [])
    return out


def _brute_force(P, m, t, m_b, m_w, m_limit):
    seqs = [q for q in _stage_sequences(m) if S.peak_memory(q, m_b, m_w) <= m_limit]
    best = None
    for combo in itertools.product(seqs, repeat=P):
        try:
            ms = S.simulate(list(combo), t).makespan
        except RuntimeError:
            continue
        best = ms if best is None else min(best, ms)
    return best


@pytest.mark.parametrize("case", [
    (2, 2, EQUAL, 4), (2, 2, EQUAL, 8), (2, 3, EQUAL, 4), (2, 3, EQUAL, 8),
    (2, 3, {"F": 2, "B": 3, "W": 1}, 4), (2, 3, {"F": 2, "B": 3, "W": 1}, 8),
    (3, 2, EQUAL, 6), (3, 2, {"F": 1, "B": 2, "W": 1}, 12), (2, 4, EQUAL, 4),
])
def test_optimal_on_tiny_pipelines(case):
    P, m, t, m_limit = case
    opt = _brute_force(P, m, t, 2, 1, m_limit)
    _, ms, _, _ = H.schedule(P, m, t, 2, 1, m_limit)
    assert ms == opt

