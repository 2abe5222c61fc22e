"""Pins for the oracle's schedule model against what the pages fix.

* [ZB] Table 2 bubble sizes: 1F1B (p-1)(T_F+T_B+T_W), ZB-H1 (p-1)(T_F+T_B-T_W),
  ZB-H2 (p-1)(T_F+T_B-2T_W) (the handcrafted orders assume T_W <= T_F).
* [TUT] 1F1B/GPipe bubble (P-1)/(m+P-1); the interleaved table (golden file).
* [ZB] peak memories: 1F1B P*M_B on the first stage, (P-s)M_B + s M_W on stage s
  for ZB-H1, (2P-1)M_B for ZB-H2's first stage.
* [AUD] worked two-stage schedule and its rejection cases (golden file).
"""
import json
import os
from fractions import Fraction

import pytest

from oracle import schedules as sch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

TIMES = [(1, 1, 1), (2, 3, 1), (3, 4, 2), (2, 2, 1), (3, 1, 2), (2, 1, 1), (5, 7, 3), (4, 4, 3)]


@pytest.mark.parametrize("P", [2, 4, 8, 16])
@pytest.mark.parametrize("tfbw", TIMES)
def test_table2_bubble_closed_forms(P, tfbw):
    F, B, W = tfbw
    t = dict(F=F, B=B, W=W)
    m = 3 * P
    assert sch.simulate(sch.stage_orders("1f1b", P, m), t).bubble == (P - 1) * (F + B + W)
    assert sch.simulate(sch.stage_orders("gpipe", P, m), t).bubble == (P - 1) * (F + B + W)
    assert sch.simulate(sch.stage_orders("zbh1", P, m), t).bubble == (P - 1) * (F + B - W)
    assert sch.simulate(sch.stage_orders("zbh2", P, m), t).bubble == max(0, (P - 1) * (F + B - 2 * W))


@pytest.mark.parametrize("P,m", [(4, 8), (8, 8), (8, 16), (2, 4), (3, 7)])
def test_1f1b_bubble_fraction(P, m):
    r = sch.simulate(sch.stage_orders("1f1b", P, m), dict(F=1, B=1, W=1))
    assert r.bubble_rate == Fraction(P - 1, m + P - 1)


def test_bubble_p4_m8_is_27_3_percent():
    r = sch.simulate(sch.stage_orders("1f1b", 4, 8), dict(F=1, B=1, W=1))
    assert r.bubble_rate == Fraction(3, 11)
    assert round(100 * float(r.bubble_rate), 1) == 27.3


def test_interleaved_table_golden():
    g = json.load(open(os.path.join(GOLDEN, "tut_interleaved_bubble_table.json")))
    for row in g["rows"]:
        for v in (1, 2, 4):
            r = sch.simulate_interleaved(row["P"], row["m"], v, dict(F=1, B=1, W=1))
            assert r.bubble_rate == Fraction(row["P"] - 1, v * row["m"] + row["P"] - 1)
            assert round(100 * float(r.bubble_rate), 1) == row["v%d" % v]


def test_zbh2_zero_bubble_but_global_span_ratio_differs():
    r = sch.simulate(sch.stage_orders("zbh2", 4, 8), dict(F=1, B=1, W=1))
    assert r.bubble == 0
    # every stage is busy for 24 slots but stages start 0..3 slots apart
    assert r.global_ratio(4) == 1 - Fraction(96, 4 * 27)


def test_zbh2_first_stage_runs_seven_forwards_before_first_b():
    """[ZB] ZB-H2 example, p = 4, m = 8: microbatches 1-7 forward before the first B."""
    o = sch.order_zbh2(4, 8, 0)
    first_b = next(i for i, (k, _) in enumerate(o) if k == "B")
    assert first_b == 7 and all(k == "F" for k, _ in o[:7])


def test_warmup_counts():
    """[ZB] ZB-H1 / 1F1B: stage i (1-indexed) runs p - i + 1 forwards before its first B."""
    P, m = 6, 12
    for name in ("1f1b", "zbh1"):
        for s in range(P):
            o = sch.ORDERS[name](P, m, s)
            first_b = next(i for i, (k, _) in enumerate(o) if k in "BU")
            assert first_b == P - s


@pytest.mark.parametrize("P", [2, 4, 8])
@pytest.mark.parametrize("mb,mw", [(7, 5), (1000, 1), (3, 3)])
def test_peak_memory_closed_forms(P, mb, mw):
    m = 3 * P
    assert sch.peak_memory(sch.order_1f1b(P, m, 0), mb, mw) == P * mb
    for s in range(P):
        assert sch.peak_memory(sch.order_1f1b(P, m, s), mb, mw) == (P - s) * mb
        assert sch.peak_memory(sch.order_zbh1(P, m, s), mb, mw) == (P - s) * mb + s * mw
    assert sch.peak_memory(sch.order_zbh2(P, m, 0), mb, mw) == (2 * P - 1) * mb


def test_every_order_releases_all_memory_and_is_valid():
    for name in ("gpipe", "1f1b", "zbh1", "zbh2", "wlast"):
        for P, m in ((2, 4), (4, 8), (8, 24), (8, 32)):
            orders = sch.stage_orders(name, P, m)
            for o in orders:
                assert sch.memory_profile(o, 5, 3)[-1] == 0
            r = sch.simulate(orders, dict(F=1, B=1, W=1))
            lin = sch.linearize(orders, r)
            assert sch.validate_linear(P, m, lin) == (sch.OK, -1)


def test_w_order_ascending_per_stage():
    for name in ("zbh1", "zbh2", "wlast"):
        for s in range(4):
            ws = [j for k, j in sch.ORDERS[name](4, 8, s) if k == "W"]
            assert ws == list(range(8))


def test_profiled_times_keep_the_pages_ordering():
    """With the pages' profiled pass times (Table 9, integer microseconds) the
    handcrafted bubbles order as 1F1B > ZB-H1 > ZB-H2, as Table 5 reports."""
    g = json.load(open(os.path.join(GOLDEN, "zb_table9_profiled_times.json")))
    for row in g["rows"]:
        t = {k: int(round(1000 * row["T_" + k])) for k in "FBW"}
        P, m = 8, row["m"]
        b = [sch.simulate(sch.stage_orders(n, P, m), t).bubble for n in ("1f1b", "zbh1", "zbh2")]
        assert b[0] > b[1] > b[2] >= 0


def test_audit_worked_schedule_golden():
    g = json.load(open(os.path.join(GOLDEN, "aud_worked_schedule.json")))
    r = sch.inspect_events(g["tasks"], g["stage_count"])
    assert r["span"] == g["expect"]["span"]
    assert r["unfinished_activations"] == g["expect"]["unfinished_activations"]
    assert 0 <= r["bubble_ratio"] < g["expect"]["bubble_ratio_below"]
    assert r["bubble_ratio"] == Fraction(*g["expect"]["bubble_ratio_exact"])
    for case in g["rejections"]:
        with pytest.raises(sch.ScheduleError, match=case["error"]):
            sch.inspect_events(g["tasks"] + [case["extra"]], g["stage_count"])
    assert sch.inspect_events(list(g["tasks"]), 2) == r
    with pytest.raises(sch.ScheduleError, match="invalid_stage_count"):
        sch.inspect_events(g["tasks"], 0)
    with pytest.raises(sch.ScheduleError, match="invalid_stage"):
        sch.inspect_events(g["tasks"], 1)  # the tasks of stage 1 name an unknown stage
    # every F is released by its W: stage 0 holds two activations at once (F0, F1 before W0)
    assert r["peak_live_activations"] == 2
    bad = [dict(t) for t in g["tasks"]]
    bad[3]["depends_on"] = ["nope"]
    with pytest.raises(sch.ScheduleError, match="missing_dependency"):
        sch.inspect_events(bad, 2)
    bad = [dict(t) for t in g["tasks"]]
    bad[0]["end"] = 0
    with pytest.raises(sch.ScheduleError, match="invalid_interval"):
        sch.inspect_events(bad, 2)


def test_validator_cases():
    P, m = 2, 2
    good = [(0, "F", 0), (1, "F", 0), (1, "B", 0), (0, "B", 0), (0, "F", 1), (1, "F", 1),
            (1, "W", 0), (1, "B", 1), (0, "B", 1), (0, "W", 0), (0, "W", 1), (1, "W", 1)]
    assert sch.validate_linear(P, m, good) == (sch.OK, -1)
    assert sch.validate_linear(P, m, good + [(0, "W", 1)]) == (sch.E_DUPLICATE, 12)
    assert sch.validate_linear(P, m, good[:-1]) == (sch.E_MISSING, 11)
    assert sch.validate_linear(P, m, [(2, "F", 0)] + good) == (sch.E_INVALID_STAGE, 0)
    assert sch.validate_linear(P, m, [(0, "F", 2)] + good) == (sch.E_INVALID_MB, 0)
    assert sch.validate_linear(P, m, [(0, "X", 0)] + good) == (sch.E_ARG, 0)
    # B on stage 0 before B on stage 1
    swapped = list(good)
    swapped[2], swapped[3] = swapped[3], swapped[2]
    assert sch.validate_linear(P, m, swapped) == (sch.E_DEPENDENCY, 2)
    # F on stage 1 before stage 0
    assert sch.validate_linear(P, m, [(1, "F", 0)] + good) == (sch.E_DEPENDENCY, 0)
    # W before its B
    wb = [(0, "F", 0), (1, "F", 0), (1, "W", 0)]
    assert sch.validate_linear(P, m, wb) == (sch.E_DEPENDENCY, 2)
    # unsplit plus split of one pass is a duplicate
    u = [(0, "F", 0), (1, "F", 0), (1, "U", 0), (1, "W", 0)]
    assert sch.validate_linear(P, m, u) == (sch.E_DUPLICATE, 3)


def test_inspector_ledger_counts_w_stash():
    """An activation stays held from F through B until its W: dropping the W of
    one microbatch leaves one unfinished activation; a B alone releases nothing."""
    g = json.load(open(os.path.join(GOLDEN, "aud_worked_schedule.json")))
    no_w = [t for t in g["tasks"] if t["id"] != "s1w1"]
    assert sch.inspect_events(no_w, 2)["unfinished_activations"] == 1
    only_f = [t for t in g["tasks"] if t["kind"] == "F"]
    assert sch.inspect_events(only_f, 2)["unfinished_activations"] == 4


def test_inspector_reports_earliest_violation():
    """Two consumers start too early; the one with the earlier start is named.
    Two overlaps on one stage; the later-starting member of the earliest pair."""
    base = [{"id": "p", "stage": 0, "micro": 0, "kind": "F", "start": 0, "end": 4}]
    late = {"id": "c1", "stage": 1, "micro": 0, "kind": "F", "start": 3, "end": 5, "depends_on": ["p"]}
    early = {"id": "c2", "stage": 2, "micro": 0, "kind": "F", "start": 1, "end": 2, "depends_on": ["p"]}
    with pytest.raises(sch.ScheduleError) as e:
        sch.inspect_events(base + [late, early], 3)
    assert e.value.args == ("dependency_violation", 2)
    ov = [{"id": i, "stage": 0, "micro": 0, "kind": "W", "start": s, "end": s + 2} for i, s in
          (("a", 5), ("b", 0), ("c", 6), ("d", 1))]
    with pytest.raises(sch.ScheduleError) as e:
        sch.inspect_events(ov, 1)
    assert e.value.args == ("stage_overlap", 3)  # d (start 1) overlaps b (start 0)
