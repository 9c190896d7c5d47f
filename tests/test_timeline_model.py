"""The timeline accounting (idle-CU fraction, phase rates) and the crew model,
pinned to the worked example the KOSMOS explainer prints ("A worked example"
paragraph; tests/golden/worked_example.json) -- CPU only."""
import json
import os

import pytest

from gemm_collective_persistent_amd.timeline import crew_model, phase_rate, summarize

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "worked_example.json")


@pytest.fixture(scope="module")
def ex():
    with open(GOLDEN) as f:
        return json.load(f)


def test_crew_model_reproduces_the_printed_numbers(ex):
    t_fixed, t_switch, sp = crew_model(ex["gemm_full_ms"], ex["throughput_fraction_on_rest"],
                                       ex["tail_fixed_ms"], ex["tail_switching_ms"])
    # the page rounds 10 / 0.93 to 10.75 ms and adds the tails to it
    assert t_fixed - ex["tail_fixed_ms"] == pytest.approx(ex["gemm_on_rest_ms"], abs=0.01)
    assert t_fixed == pytest.approx(ex["total_fixed_ms"], abs=0.01)
    assert t_switch == pytest.approx(ex["total_switching_ms"], abs=0.01)
    assert abs(sp - ex["speedup"]) <= ex["speedup_rounding"]
    # no tail saved, no gain; a crew that costs nothing (fraction 1) leaves the GEMM time
    assert crew_model(10.0, 0.93, 1.5, 1.5)[2] == 1.0
    assert crew_model(10.0, 1.0, 0.0, 0.0)[:2] == (10.0, 10.0)


def _wg(begin, end, recs):
    return (0, begin, end, recs)


def _example_timelines(ex, scale=1000.0):
    """Per-workgroup timelines of the two schedules of the worked example, in
    microseconds: 224 builders busy for the GEMM on the remaining units, a
    crew of 32 communicating for the whole call, and a reduction tail that
    the crew does alone (fixed) or that every workgroup shares (switching)."""
    n, crew = ex["cus_total"], ex["cus_reserved"]
    g = ex["gemm_on_rest_ms"] * scale
    tf, ts = ex["tail_fixed_ms"] * scale, ex["tail_switching_ms"] * scale
    fixed, switch = [], []
    for w in range(n):
        if w < crew:
            fixed.append(_wg(0.0, g + tf, [("reduce", w, 0.0, g + tf)]))
            switch.append(_wg(0.0, g + ts, [("reduce", w, 0.0, g + ts)]))
        else:
            fixed.append(_wg(0.0, g + tf, [("tile", w, 0.0, g)]))          # idle through the tail
            switch.append(_wg(0.0, g + ts, [("tile", w, 0.0, g), ("reduce", w, g, g + ts)]))
    return fixed, switch


def test_summarize_matches_the_closed_form(ex):
    fixed, switch = _example_timelines(ex)
    n, crew = ex["cus_total"], ex["cus_reserved"]
    sf, ss = summarize(fixed), summarize(switch)
    assert sf["span_us"] == pytest.approx(ex["total_fixed_ms"] * 1000.0)
    assert ss["span_us"] == pytest.approx(ex["total_switching_ms"] * 1000.0)
    # fixed: the 224 builders idle through the 1.5 ms tail
    idle = (n - crew) * ex["tail_fixed_ms"] / (n * ex["total_fixed_ms"])
    assert sf["idle_frac"] == pytest.approx(idle, abs=1e-4)
    assert ss["idle_frac"] == pytest.approx(0.0, abs=1e-4)
    assert sf["span_us"] / ss["span_us"] == pytest.approx(ex["speedup"], abs=ex["speedup_rounding"])
    assert sf["kinds"]["tile"]["n"] == n - crew and ss["kinds"]["reduce"]["n"] == n


def test_summarize_counts_gaps_between_launches():
    """Two launches of 4 workgroups, each busy 10 us, 5 us apart: the gap is
    idle for every compute unit."""
    tl = [_wg(0.0, 10.0, [("move", 0, 0.0, 10.0)]) for _ in range(4)]
    tl += [_wg(15.0, 25.0, [("tile", 0, 15.0, 25.0)]) for _ in range(4)]
    s = summarize(tl, workgroups=4)
    assert s["span_us"] == pytest.approx(25.0)
    assert s["idle_frac"] == pytest.approx(5.0 / 25.0)
    # read as one launch of 8 workgroups the same records would be 60% idle
    assert summarize(tl)["idle_frac"] == pytest.approx(1.0 - 80.0 / (8 * 25.0))


def test_phase_rate():
    tl = [_wg(0.0, 20.0, [("move", 0, 2.0, 6.0), ("tile", 1, 6.0, 20.0)]),
          _wg(0.0, 20.0, [("move", 1, 3.0, 12.0)])]
    r = phase_rate(tl, "move", 1e6)     # 1 MB over 2..12 us
    assert r["span_us"] == pytest.approx(10.0)
    assert r["gb_s"] == pytest.approx(100.0)
    assert phase_rate(tl, "reduce", 1.0)["gb_s"] is None
