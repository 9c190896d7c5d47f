"""Summary of a persistent kernel's timeline (``Workspace.trace``).

The idle-CU fraction is the share of compute-unit time, over the call's span
(first workgroup start to last workgroup exit, across every launch the call
made) times the workgroups one launch holds (one per compute unit), that no
piece of work covers: time spent polling ready counters, claiming entries,
waiting at the start or after leaving while others still run, and -- for
the unfused baselines -- the gaps between their launches.
"""
from __future__ import annotations


def summarize(timeline, workgroups: int | None = None) -> dict:
    """`timeline`: the list ``Workspace.trace(grid, launches=L)`` returns (one
    entry per workgroup and launch).  `workgroups`: the grid of one launch
    (default: every entry is a workgroup of a single launch)."""
    if not timeline:
        raise ValueError("empty timeline")
    t_begin = min(b for _, b, _, _ in timeline)
    t_end = max(e for _, _, e, _ in timeline)
    span = max(t_end - t_begin, 1e-9)
    n_wg = len(timeline) if workgroups is None else int(workgroups)
    kinds: dict = {}
    work = wait = 0.0
    for _, _, _, recs in timeline:
        for kind, _, t0, t1 in recs:
            d = t1 - t0
            k = kinds.setdefault(kind, {"n": 0, "us": 0.0, "first_us": t0 - t_begin, "last_us": t1 - t_begin})
            k["n"] += 1
            k["us"] += d
            k["first_us"] = min(k["first_us"], t0 - t_begin)
            k["last_us"] = max(k["last_us"], t1 - t_begin)
            if kind == "wait":
                wait += d
            else:
                work += d
    for k in kinds.values():
        k["mean_us"] = k["us"] / k["n"]
        for f in ("us", "mean_us", "first_us", "last_us"):
            k[f] = round(k[f], 2)
    total = n_wg * span
    return {"span_us": round(span, 2), "workgroups": n_wg, "idle_frac": round(1.0 - work / total, 4),
            "wait_frac": round(wait / total, 4), "kinds": kinds}


def phase_rate(timeline, kind: str, nbytes: float) -> dict:
    """Bytes per second of the pieces of work of one kind (a mover or reducer
    phase): `nbytes` moved by all of them over the phase's span (first start
    to last end of that kind), in GB/s, with the span in microseconds."""
    t0 = [r[2] for _, _, _, recs in timeline for r in recs if r[0] == kind]
    t1 = [r[3] for _, _, _, recs in timeline for r in recs if r[0] == kind]
    if not t0:
        return {"span_us": 0.0, "gb_s": None}
    span = max(max(t1) - min(t0), 1e-9)
    return {"span_us": round(span, 2), "gb_s": round(nbytes / (span * 1e-6) / 1e9, 1)}


def crew_model(t_gemm_full, frac_on_rest, tail_fixed, tail_switch):
    """The explainer's worked example ("A worked example" paragraph of the
    KOSMOS explainer page) as a model: a GEMM that takes `t_gemm_full` on the
    whole GPU keeps `frac_on_rest` of its throughput on the compute units left
    after a communication crew is reserved, and the reduction then needs
    `tail_fixed` more with the builders idle, or `tail_switch` when they join
    it.  Returns (t_fixed, t_switch, speedup)."""
    t_rest = t_gemm_full / frac_on_rest
    t_fixed = t_rest + tail_fixed
    t_switch = t_rest + tail_switch
    return t_fixed, t_switch, t_fixed / t_switch
