"""The native schedule layer (libzb.so, host code only) against the oracle.

Bit-exact on pass orders, simulated statistics, one-device linearization,
validator verdicts (crafted and randomly perturbed orders), memory peaks and
the audit page's timed-event checks.  No GPU is touched.
"""
import json
import os
import random
from fractions import Fraction

import pytest

import split_backward_gemms_amd as zb
from oracle import schedules as sch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

NAMES = ["gpipe", "1f1b", "zbh1", "zbh2", "wlast"]
CASES = [(2, 4), (4, 8), (4, 16), (8, 24), (8, 32), (3, 7), (1, 3)]
TIMES = [(1, 1, 1), (2, 3, 1), (3, 4, 2), (5, 7, 3), (1, 2, 2)]

ORACLE_STATUS = {sch.OK: zb.ZB_OK, sch.E_ARG: zb.ZB_E_ARG, sch.E_DUPLICATE: zb.ZB_E_DUPLICATE,
                 sch.E_INVALID_STAGE: zb.ZB_E_INVALID_STAGE, sch.E_INVALID_MB: zb.ZB_E_INVALID_MB,
                 sch.E_MISSING: zb.ZB_E_MISSING, sch.E_DEPENDENCY: zb.ZB_E_DEPENDENCY}


@pytest.mark.parametrize("name", NAMES)
@pytest.mark.parametrize("P,m", CASES)
def test_stage_orders_match_oracle(name, P, m):
    if name == "zbh2" and m < 2 * P - 1:
        with pytest.raises(zb.ZbError):
            zb.zb_schedule_stage_order(name, P, m, 0)
        return
    for s in range(P):
        native = [(k, j) for _, k, j in zb.zb_schedule_stage_order(name, P, m, s)]
        assert native == sch.ORDERS[name](P, m, s)


@pytest.mark.parametrize("name", NAMES)
@pytest.mark.parametrize("P,m", CASES)
@pytest.mark.parametrize("t", TIMES)
def test_simulation_and_linearization_bit_exact(name, P, m, t):
    if name == "zbh2" and m < 2 * P - 1:
        return
    lin, st = zb.zb_schedule_build(name, P, m, t)
    orders = sch.stage_orders(name, P, m)
    r = sch.simulate(orders, dict(F=t[0], B=t[1], W=t[2]))
    assert lin == sch.linearize(orders, r)
    assert (st["makespan"], st["span"], st["busy"], st["ideal"], st["bubble"]) == (
        r.makespan, r.span, r.busy, r.ideal, r.bubble)


def test_simulate_with_comm_matches_oracle():
    for name in ("1f1b", "zbh1", "zbh2"):
        orders = sch.stage_orders(name, 4, 8)
        flat = [(s, k, j) for s, o in enumerate(orders) for k, j in o]
        lin, start, end, st = zb.zb_schedule_simulate(4, 8, flat, (3, 4, 2), t_comm=1)
        r = sch.simulate(orders, dict(F=3, B=4, W=2), t_comm=1)
        assert lin == sch.linearize(orders, r)
        assert [r.start[(s, k, j)] for s, k, j in lin] == start
        assert [r.end[(s, k, j)] for s, k, j in lin] == end
        assert st["makespan"] == r.makespan


def test_closed_forms_native():
    assert zb.zb_schedule_build("1f1b", 4, 8)[1]["bubble"] == 9  # (P-1)(T_F+T_B+T_W)
    st = zb.zb_schedule_build("1f1b", 4, 8)[1]
    assert Fraction(st["bubble"], st["makespan"]) == Fraction(3, 11)
    assert zb.zb_schedule_build("zbh1", 4, 8)[1]["bubble"] == 3
    assert zb.zb_schedule_build("zbh2", 4, 8)[1]["bubble"] == 0


def test_interleaved_table_native():
    g = json.load(open(os.path.join(GOLDEN, "tut_interleaved_bubble_table.json")))
    for row in g["rows"]:
        for v in (1, 2, 4):
            st = zb.zb_schedule_simulate_interleaved(row["P"], row["m"], v)
            rate = Fraction(st["bubble"], st["makespan"])
            assert rate == Fraction(row["P"] - 1, v * row["m"] + row["P"] - 1)
            assert round(100 * float(rate), 1) == row["v%d" % v]


def _perturb(ops, rng):
    ops = list(ops)
    r = rng.random()
    if r < 0.3 and len(ops) > 1:
        i, j = rng.randrange(len(ops)), rng.randrange(len(ops))
        ops[i], ops[j] = ops[j], ops[i]
    elif r < 0.45:
        del ops[rng.randrange(len(ops))]
    elif r < 0.6:
        ops.insert(rng.randrange(len(ops) + 1), ops[rng.randrange(len(ops))])
    elif r < 0.7:
        i = rng.randrange(len(ops))
        s, k, j = ops[i]
        ops[i] = (s + rng.choice([-9, 9]), k, j)
    elif r < 0.8:
        i = rng.randrange(len(ops))
        s, k, j = ops[i]
        ops[i] = (s, k, j + rng.choice([-5, 50]))
    elif r < 0.85:
        i = rng.randrange(len(ops))
        s, k, j = ops[i]
        ops[i] = (s, rng.choice("XUB"), j)
    else:
        i = rng.randrange(len(ops) - 1) if len(ops) > 1 else 0
        ops[i:i + 2] = ops[i:i + 2][::-1]
    return ops


def test_validator_matches_oracle_on_perturbed_orders():
    rng = random.Random(1234)
    for trial in range(1500):
        name = rng.choice(NAMES)
        P, m = rng.choice([(2, 4), (3, 5), (4, 8)])
        if name == "zbh2" and m < 2 * P - 1:
            name = "zbh1"
        lin, _ = zb.zb_schedule_build(name, P, m)
        ops = lin
        for _ in range(rng.randint(0, 3)):
            ops = _perturb(ops, rng)
        want = sch.validate_linear(P, m, ops)
        got = zb.zb_schedule_validate(P, m, ops)
        assert got == (ORACLE_STATUS[want[0]], want[1]), (trial, name, P, m)


def test_validator_good_orders_and_empty():
    for name in NAMES:
        lin, _ = zb.zb_schedule_build(name, 4, 8)
        assert zb.zb_schedule_validate(4, 8, lin) == (zb.ZB_OK, -1)
    st, bad = zb.zb_schedule_validate(2, 2, [])
    assert st == zb.ZB_E_MISSING and bad == 0


@pytest.mark.parametrize("P", [2, 4, 8])
def test_peak_memory_native(P):
    m = 3 * P
    for name in ("1f1b", "zbh1", "zbh2"):
        lin, _ = zb.zb_schedule_build(name, P, m)
        for s in range(P):
            got = zb.zb_schedule_peak_memory(lin, s, 7, 5)
            assert got == sch.peak_memory(sch.ORDERS[name](P, m, s), 7, 5)
    lin, _ = zb.zb_schedule_build("zbh2", P, m)
    assert zb.zb_schedule_peak_memory(lin, 0, 7, 5) == (2 * P - 1) * 7


def test_events_inspect_audit_golden():
    g = json.load(open(os.path.join(GOLDEN, "aud_worked_schedule.json")))
    st, rep, bad = zb.zb_events_inspect(g["tasks"], g["stage_count"])
    assert st == zb.ZB_OK
    assert rep["span"] == 8 and rep["unfinished_activations"] == 0
    assert rep["bubble_ratio"] == 0.25
    want = {"duplicate_task": zb.ZB_E_DUPLICATE, "invalid_stage": zb.ZB_E_INVALID_STAGE,
            "stage_overlap": zb.ZB_E_OVERLAP, "dependency_violation": zb.ZB_E_DEPENDENCY}
    for case in g["rejections"]:
        st, _, _ = zb.zb_events_inspect(g["tasks"] + [case["extra"]], 2)
        assert st == want[case["error"]]
    assert zb.zb_events_inspect(g["tasks"], 0)[0] == zb.ZB_E_ARG
    assert zb.zb_events_inspect(g["tasks"], 1)[0] == zb.ZB_E_INVALID_STAGE
    assert rep["peak_live_activations"] == 2
    bad_dep = [dict(t) for t in g["tasks"]]
    bad_dep[3]["depends_on"] = ["nope"]
    assert zb.zb_events_inspect(bad_dep, 2)[0] == zb.ZB_E_MISSING
    bad_iv = [dict(t) for t in g["tasks"]]
    bad_iv[0]["end"] = 0
    assert zb.zb_events_inspect(bad_iv, 2)[0] == zb.ZB_E_INTERVAL


def test_events_inspect_matches_oracle_on_simulated_schedules():
    """A simulated schedule, exported as timed events with its dependency edges,
    passes both inspectors with the same span and ratio."""
    for name in ("1f1b", "zbh1", "zbh2"):
        P, m = 4, 8
        orders = sch.stage_orders(name, P, m)
        r = sch.simulate(orders, dict(F=2, B=3, W=1))
        tasks = []
        for s, o in enumerate(orders):
            for k, j in o:
                deps = []
                if k == "F" and s > 0:
                    deps.append(f"{s-1}F{j}")
                if k in "BU" and s < P - 1:
                    deps.append(f"{s+1}{'U' if name == '1f1b' else 'B'}{j}")
                if k == "W":
                    deps.append(f"{s}B{j}")
                tasks.append({"id": f"{s}{k}{j}", "stage": s, "micro": j, "kind": k,
                              "start": r.start[(s, k, j)], "end": r.end[(s, k, j)], "depends_on": deps})
        want = sch.inspect_events(tasks, P)
        st, got, _ = zb.zb_events_inspect(tasks, P)
        assert st == zb.ZB_OK
        assert got["span"] == want["span"] and got["busy"] == want["busy"]
        assert abs(got["bubble_ratio"] - float(want["bubble_ratio"])) < 1e-12
        assert got["unfinished_activations"] == want["unfinished_activations"] == 0
        assert got["peak_live_activations"] == want["peak_live_activations"]


_INSPECT_STATUS = {"invalid_stage_count": zb.ZB_E_ARG, "duplicate_task": zb.ZB_E_DUPLICATE,
                   "invalid_stage": zb.ZB_E_INVALID_STAGE, "invalid_interval": zb.ZB_E_INTERVAL,
                   "missing_dependency": zb.ZB_E_MISSING, "dependency_violation": zb.ZB_E_DEPENDENCY,
                   "stage_overlap": zb.ZB_E_OVERLAP}


def _timed_tasks(name, P, m, t):
    orders = sch.stage_orders(name, P, m)
    r = sch.simulate(orders, t)
    tasks = []
    for s, o in enumerate(orders):
        for k, j in o:
            deps = []
            if k == "F" and s > 0:
                deps.append(f"{s-1}F{j}")
            if k in "BU":
                deps.append(f"{s}F{j}")
                if s < P - 1:
                    deps.append(f"{s+1}{'U' if k == 'U' else 'B'}{j}")
            if k == "W":
                deps.append(f"{s}B{j}")
            tasks.append({"id": f"{s}{k}{j}", "stage": s, "micro": j, "kind": k,
                          "start": r.start[(s, k, j)], "end": r.end[(s, k, j)], "depends_on": deps})
    return tasks


def test_events_inspect_matches_oracle_on_perturbed_schedules():
    """Both inspectors give the same verdict, offending event and report on
    simulated schedules with random faults planted: moved or shortened events,
    repeated ids, wrong stages, dropped or renamed dependencies, removed W's."""
    rng = random.Random(2027)
    seen = set()
    for trial in range(1500):
        name = rng.choice(["1f1b", "zbh1", "zbh2", "gpipe"])
        P = rng.randint(2, 4)
        m = rng.randint(2 * P - 1, 2 * P + 2) if name == "zbh2" else rng.randint(1, 6)
        t = dict(F=rng.randint(1, 3), B=rng.randint(1, 3), W=rng.randint(1, 2))
        tasks = _timed_tasks(name, P, m, t)
        for _ in range(rng.randint(0, 3)):
            i = rng.randrange(len(tasks))
            x = dict(tasks[i])
            fault = rng.randrange(8)
            if fault == 0:
                x["start"] = max(0, x["start"] - rng.randint(1, 3))
            elif fault == 1:
                x["end"] = x["start"] - rng.choice([0, 1])
            elif fault == 2:
                x["id"] = tasks[rng.randrange(len(tasks))]["id"]
            elif fault == 3:
                x["stage"] = rng.choice([-1, P, P + 1])
            elif fault == 4:
                x["depends_on"] = list(x["depends_on"]) + ["nobody"]
            elif fault == 5:
                x["start"] += rng.randint(1, 4)
                x["end"] += rng.randint(1, 4)
            elif fault == 6 and x["kind"] == "W":
                tasks.pop(i)
                continue
            else:
                x["stage"] = rng.randrange(P)
            tasks[i] = x
        count = rng.choice([P, P, P, 0])
        try:
            want = sch.inspect_events(tasks, count)
            w_st, w_bad = zb.ZB_OK, -1
        except sch.ScheduleError as e:
            want = None
            w_st = _INSPECT_STATUS[e.args[0]]
            w_bad = e.args[1] if len(e.args) > 1 else -1
        st, got, bad = zb.zb_events_inspect(tasks, count)
        assert (st, bad) == (w_st, w_bad), (trial, st, bad, w_st, w_bad)
        seen.add(st)
        if want is not None:
            assert got["span"] == want["span"] and got["busy"] == want["busy"]
            assert abs(got["bubble_ratio"] - float(want["bubble_ratio"])) < 1e-12
            assert got["unfinished_activations"] == want["unfinished_activations"]
            assert got["peak_live_activations"] == want["peak_live_activations"]
    assert seen >= set(_INSPECT_STATUS.values()) | {zb.ZB_OK}


# ------------------------------------------------ automatic (heuristic) scheduler

def test_heuristic_matches_oracle():
    from oracle import heuristic as heu
    rng = random.Random(11)
    for _ in range(300):
        P, m = rng.randint(1, 6), rng.randint(1, 12)
        t = {"F": rng.randint(1, 5), "B": rng.randint(1, 6), "W": rng.randint(1, 4)}
        m_b, m_w = rng.randint(1, 5), rng.randint(1, 5)
        m_limit = rng.randint(max(m_b, m_w), (2 * P + 1) * m_b + m_w)
        comm = rng.choice([0, 0, 1, 2])
        orders, ms, fill, balance = heu.schedule(P, m, t, m_b, m_w, m_limit, comm)
        sim = sch.simulate(orders, t, comm)
        ops, st, choice = zb.zb_schedule_heuristic(P, m, (t["F"], t["B"], t["W"]), m_b, m_w, m_limit, comm)
        assert ops == sch.linearize(orders, sim)
        assert st["makespan"] == ms
        assert choice == (fill, balance)


@pytest.mark.parametrize("P,m", [(4, 8), (8, 24)])
def test_heuristic_order_runs_through_validator(P, m):
    for lim in (P * 2, 2 * P * 2):
        ops, st, _ = zb.zb_schedule_heuristic(P, m, (1, 1, 1), 2, 1, lim)
        assert zb.zb_schedule_validate(P, m, ops) == (zb.ZB_OK, -1)
        for s in range(P):
            assert zb.zb_schedule_peak_memory(ops, s, 2, 1) <= lim


def test_heuristic_rejects_small_budget():
    with pytest.raises(zb.ZbError):
        zb.zb_schedule_heuristic(4, 8, (1, 1, 1), 2, 3, 2)
    with pytest.raises(zb.ZbError):
        zb.zb_schedule_heuristic(0, 8, (1, 1, 1), 2, 1, 8)


# ------------------------------------------------------------------- ZB-V

def test_zbv_matches_oracle():
    from oracle import vshape as vs
    rng = random.Random(13)
    for _ in range(300):
        P, m = rng.randint(1, 6), rng.randint(1, 12)
        t = {"F": rng.randint(1, 5), "B": rng.randint(1, 6), "W": rng.randint(1, 4)}
        m_b, m_w = rng.randint(1, 5), rng.randint(1, 5)
        m_limit = max(m_w, rng.randint(2 * m_b + max(0, m_w - m_b), 3 * P * m_b + m_w))
        comm = rng.choice([0, 0, 1, 2])
        orders = vs.build(P, m, t, m_b, m_w, m_limit, comm)
        sim = vs.simulate(P, orders, t, comm)
        ops, st = zb.zb_schedule_zbv(P, m, (t["F"], t["B"], t["W"]), m_b, m_w, m_limit, comm)
        assert ops == vs.linearize(orders, sim)
        assert (st["makespan"], st["ideal"], st["bubble"]) == (sim.makespan, sim.ideal, sim.bubble)
        assert zb.zb_schedule_validate(2 * P, m, ops) == (zb.ZB_OK, -1)


def test_zbv_equal_times_matches_oracle():
    """At equal pass times both sides search for a zero-bubble order and keep
    the better of it and the list order: same orders, same statistics."""
    from oracle import vshape as vs
    rng = random.Random(17)
    for _ in range(60):
        P = rng.randint(1, 5)
        m = rng.randint(1, 4 * P)
        tt = rng.randint(1, 4)
        t = {"F": tt, "B": tt, "W": tt}
        m_b, m_w = rng.randint(1, 4), rng.randint(1, 4)
        lo = 2 * m_b + max(0, m_w - m_b)
        m_limit = max(m_w, rng.choice([lo, 2 * P * max(m_b, m_w), rng.randint(lo, 3 * P * max(m_b, m_w))]))
        comm = rng.choice([0, 0, 0, 1])
        orders = vs.build(P, m, t, m_b, m_w, m_limit, comm)
        sim = vs.simulate(P, orders, t, comm)
        ops, st = zb.zb_schedule_zbv(P, m, (tt, tt, tt), m_b, m_w, m_limit, comm)
        assert ops == vs.linearize(orders, sim)
        assert (st["makespan"], st["ideal"], st["bubble"]) == (sim.makespan, sim.ideal, sim.bubble)


@pytest.mark.parametrize("P,m", [(2, 4), (4, 8), (4, 32), (6, 18), (7, 21), (8, 16), (8, 24), (8, 32), (8, 64)])
def test_zbv_zero_bubble_at_equal_times(P, m):
    """The native V order at T_F = T_B = T_W: no bubble on any device, each
    device peaking at P M_B of a whole stage (checked with the oracle's
    simulator and ledger)."""
    from oracle import vshape as vs
    ops, st = zb.zb_schedule_zbv(P, m, (1, 1, 1), 1, 1, 2 * P)
    assert st["bubble"] == 0
    assert zb.zb_schedule_validate(2 * P, m, ops) == (zb.ZB_OK, -1)
    orders = [[] for _ in range(P)]
    for c, k, j in ops:
        orders[vs.device_of(c, P)].append((k, c, j))
    sim = vs.simulate(P, orders, {"F": 1, "B": 1, "W": 1})
    assert sim.bubble == 0 and all(x == sim.ideal for x in sim.device_cost)
    assert [vs.peak_memory(o, 1, 1) for o in orders] == [2 * P] * P


def test_zbv_rejects_small_budget():
    with pytest.raises(zb.ZbError):
        zb.zb_schedule_zbv(4, 8, (1, 1, 1), 2, 3, 4)
    with pytest.raises(zb.ZbError):
        zb.zb_schedule_zbv(4, 8, (0, 1, 1), 1, 1, 8)
