"""Pins of the oracle's routing diagnostics ([QEvict] §3: selection churn
between consecutive routing events and Global LIR, the revival of windows
after a sustained absence from the full-precision set), fixed by hand."""
import pytest

import oracle as orc


def test_hand_trace_churn_and_revival():
    """gap 2; windows 0..3 are candidates at every event (tiers 0 F, 1 Q, 2 E).

    e1: F={0,1} R={0,1,2}        runs: 2->1, 3->1 (evicted)
    e2: F={0,2} R={0,1,2}        F churn 1-1/3, R churn 0; runs: 1->1, 2->0 (no revival: run 1 < 2)
    e3: F={0,2} R={0,1,2}        runs: 1->2 (sustained)
    e4: F={1,2} R={1,2}          0 evicted; 1 revives (run 2 >= 2); F churn 1-1/3, R churn 1-2/3
    """
    d = orc.RoutingDiagnostics(2)
    c1 = d.observe([0, 1, 2, 3], {0: 0, 1: 0, 2: 1, 3: 2})
    assert c1 == {"f_new": 2, "r_new": 3, "f_prev": 0, "f_overlap": 0, "r_prev": 0, "r_overlap": 0}
    c2 = d.observe([0, 1, 2], {0: 0, 1: 1, 2: 0, 3: 2})
    assert c2 == {"f_new": 2, "r_new": 3, "f_prev": 2, "f_overlap": 1, "r_prev": 3, "r_overlap": 3}
    d.observe([0, 1, 2], {0: 0, 1: 1, 2: 0, 3: 2})
    assert d.sums["sustained"] == 1 and d.sums["revived"] == 0
    c4 = d.observe([0, 1, 2], {0: 2, 1: 0, 2: 0, 3: 2})
    assert c4 == {"f_new": 2, "r_new": 2, "f_prev": 2, "f_overlap": 1, "r_prev": 3, "r_overlap": 2}
    s = d.sums
    assert (s["events"], s["pairs"], s["sustained"], s["revived"]) == (4, 3, 1, 1)
    assert s["sum_f_churn"] == pytest.approx(2 / 3 + 0.0 + 2 / 3, abs=1e-15)
    assert s["sum_r_churn"] == pytest.approx(0.0 + 0.0 + 1 / 3, abs=1e-15)


def test_gap_one_counts_every_demotion_and_stable_routing_has_no_churn():
    d = orc.RoutingDiagnostics(1)
    tiers = {0: 0, 1: 1, 2: 1}
    for _ in range(5):
        d.observe([0, 1, 2], tiers)
    # windows 1 and 2 start a run at the first event and never re-enter F
    assert d.sums["sustained"] == 2 and d.sums["revived"] == 0
    assert d.sums["sum_f_churn"] == 0.0 and d.sums["sum_r_churn"] == 0.0
    d.observe([0, 1, 2], {0: 1, 1: 0, 2: 1})
    assert d.sums["revived"] == 1 and d.sums["sustained"] == 3
