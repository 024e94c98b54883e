"""Pins for the oracle's pipeline-timeline model against the pages' worked
example (tests/golden/timeline_*.txt) and the closed form it must agree with."""
import math

import pytest

from oracle import timeline
from tests.conftest import golden_lines


def _params(fields):
    return {k: float(v) for k, v in (f.split("=") for f in fields[1:])}


def test_worked_example_summary_table():
    lines = golden_lines("timeline_iter8.txt")
    p = _params(lines[0])
    rows = timeline.summary_rows(int(p["iterations"]), p["issue"], p["latency"], p["compute"],
                                 [int(r[0]) for r in lines[1:]])
    for want, got in zip(lines[1:], rows):
        stages, makespan, speedup, issue_iv, compute_iv, util = want
        assert got["stages"] == int(stages)
        assert got["makespan"] == float(makespan)
        assert f"{got['speedup']:.2f}" == speedup
        assert f"{got['issue_iv']:.1f}" == issue_iv
        assert f"{got['compute_iv']:.1f}" == compute_iv
        assert f"{100 * got['compute_util']:.0f}" == util
    assert timeline.min_depth(p["latency"], p["compute"]) == int(p["min_depth"])
    assert f"{p['latency'] / p['compute']:.2f}" == "1.50"


def test_deeper_than_the_knee_changes_nothing():
    for s in range(3, 9):
        assert timeline.simulate(8, 1, 30, 20, s).makespan == 190


def test_longer_loop_raises_speedup():
    for iterations, stages, speedup in golden_lines("timeline_iter16.txt"):
        got = timeline.speedup(int(iterations), 1, 30, 20, int(stages))
        assert f"{got:.2f}" == speedup


def test_single_buffer_costs_latency_plus_compute_per_round():
    for n in (1, 2, 5, 13):
        for L, C in ((30, 20), (7, 11), (0, 5)):
            assert timeline.simulate(n, 1, L, C, 1).makespan == n * (L + C)


@pytest.mark.parametrize("ratio", [0.5, 1.5, 2.5, 4.0])
@pytest.mark.parametrize("stages", range(1, 9))
def test_steady_state_matches_closed_form(ratio, stages):
    compute, issue = 20.0, 1.0
    latency = ratio * compute
    n = 600
    s = timeline.simulate(n, issue, latency, compute, stages)
    # average compute-start interval over a late window of stages*10 rounds
    w = stages * 10
    measured = (s.compute_start[n - 1] - s.compute_start[n - 1 - w]) / w
    assert math.isclose(measured, timeline.steady_period(issue, latency, compute, stages), rel_tol=1e-9)


@pytest.mark.parametrize("latency,compute", [(30, 20), (10, 20), (50, 20), (80, 20), (41, 10), (5, 5)])
def test_knee_is_min_depth(latency, compute):
    # the smallest depth whose steady period reaches `compute` is 1 + ceil(L/C)
    # (issue is negligible here)
    knee = next(s for s in range(1, 64) if timeline.steady_period(0.0, latency, compute, s) <= compute)
    assert knee == timeline.min_depth(latency, compute)


def test_schedule_respects_slot_reuse_and_ordering():
    s = timeline.simulate(40, 1, 30, 20, 3)
    for i in range(40):
        assert s.ready[i] == s.issue_start[i] + 30
        assert s.compute_start[i] >= s.ready[i]
        if i:
            assert s.compute_start[i] >= s.compute_end[i - 1]
            assert s.issue_start[i] >= s.issue_start[i - 1] + 1
        if i >= 3:
            assert s.issue_start[i] >= s.compute_end[i - 3]
