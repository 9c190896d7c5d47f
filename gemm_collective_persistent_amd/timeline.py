"""Summary of a persistent kernel's timeline (``Workspace.trace``).

The idle-CU fraction is the share of workgroup-time, over the kernel's span
(first workgroup start to last workgroup exit) times the workgroup count,
that no piece of work covers: time spent polling ready counters, claiming
entries, and waiting at the start or after leaving while others still run.
"""
from __future__ import annotations


def summarize(timeline) -> dict:
    """`timeline`: the list ``Workspace.trace(grid)`` returns."""
    if not timeline:
        raise ValueError("empty timeline")
    t_begin = min(b for _, b, _, _ in timeline)
    t_end = max(e for _, _, e, _ in timeline)
    span = max(t_end - t_begin, 1e-9)
    n_wg = len(timeline)
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
