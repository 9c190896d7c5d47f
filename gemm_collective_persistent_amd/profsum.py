"""Short text summaries of rocprofv3 output, for the ``profiles/`` folder.

Two summaries:

``stats``    per-kernel launch counts and durations from a
             ``--kernel-trace --stats`` run (``*_kernel_stats.csv``).
``traffic``  HBM-side bytes per launch of one kernel from two ``--pmc`` runs
             (FETCH_SIZE, then WRITE_SIZE; both in KiB per dispatch).  Each
             counter is scaled by what it reads for the three plain 1 GiB
             elementwise passes ``bench.py --copy-calibration`` makes (1 GiB
             read and 1 GiB written each, by construction), so the figure is
             in the same units as the algorithmic byte count.  The summary
             records the kernel-source digest it was taken on; ``bench.py``
             ignores it once the kernels change.

Usage:
  python -m gemm_collective_persistent_amd.profsum stats STATS_CSV --command CMD --out FILE
  python -m gemm_collective_persistent_amd.profsum traffic FETCH_CSV WRITE_CSV --kernel SUBSTR
        --op NAME --workload NAME --digest HEX --command CMD --out FILE
"""
from __future__ import annotations

import argparse
import csv
import statistics
import sys

CALIB_BYTES = 1 << 30       # each calibration copy
CALIB_COPIES = 3            # copies bench.py --copy-calibration makes
CALIB_KERNEL = "neg_kernel"   # torch's elementwise negation, 1 GiB in and out


def _short(name: str) -> str:
    return name.replace("(anonymous namespace)", "{anon}").split("(")[0].replace("void ", "")


def stats(path: str, command: str) -> str:
    rows = list(csv.DictReader(open(path)))
    out = ["# rocprofv3 --kernel-trace --stats summary", f"command: {command}", "",
           f"{'calls':>6} {'avg_us':>10} {'min_us':>10} {'max_us':>10} {'total_%':>8}  kernel"]
    for r in rows:
        out.append(f"{int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:10.1f} {float(r['MinNs']) / 1e3:10.1f} "
                   f"{float(r['MaxNs']) / 1e3:10.1f} {float(r['Percentage']):8.2f}  {_short(r['Name'])[:110]}")
    return "\n".join(out) + "\n"


def _readings(path: str, counter: str):
    rows = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]
    rows.sort(key=lambda r: int(r["Dispatch_Id"]))
    return rows


def traffic(fetch_csv: str, write_csv: str, kernel: str, op: str, workload: str, digest: str, command: str) -> str:
    fr, wr = _readings(fetch_csv, "FETCH_SIZE"), _readings(write_csv, "WRITE_SIZE")

    def calib(rows):
        # the runtime may split one copy into several dispatches: sum the
        # large ones and compare with CALIB_COPIES x CALIB_BYTES
        big = [float(r["Counter_Value"]) * 1024 for r in rows if CALIB_KERNEL in r["Kernel_Name"]
               and float(r["Counter_Value"]) * 1024 > CALIB_BYTES / 8]
        if not big:
            raise SystemExit("no 1 GiB calibration copy found (run bench.py with --copy-calibration)")
        return CALIB_COPIES * CALIB_BYTES / sum(big)

    f_scale, w_scale = calib(fr), calib(wr)
    fk = [float(r["Counter_Value"]) * 1024 for r in fr if kernel in r["Kernel_Name"]]
    wk = [float(r["Counter_Value"]) * 1024 for r in wr if kernel in r["Kernel_Name"]]
    if not fk or not wk:
        raise SystemExit(f"kernel {kernel!r} not found")
    f_b, w_b = statistics.median(fk) * f_scale, statistics.median(wk) * w_scale
    return "\n".join([
        f"# HBM-side traffic of {op} on {workload} (rocprofv3 --pmc FETCH_SIZE, then WRITE_SIZE)",
        f"command_fetch: {command.replace('PMC', 'FETCH_SIZE')}",
        f"command_write: {command.replace('PMC', 'WRITE_SIZE')}",
        f"kernel: {kernel}",
        f"launches: {len(fk)} (fetch run), {len(wk)} (write run); medians below",
        f"calibration: {CALIB_COPIES} device copies of {CALIB_BYTES} bytes ({CALIB_KERNEL}); "
        f"fetch scale {f_scale:.4f}, write scale {w_scale:.4f}",
        f"fetch_bytes_per_launch: {f_b:.0f}",
        f"write_bytes_per_launch: {w_b:.0f}",
        f"traffic_bytes_per_launch: {f_b + w_b:.0f}",
        f"source_digest: {digest}",
    ]) + "\n"


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("--command", required=True)
    s.add_argument("--out", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("fetch_csv")
    t.add_argument("write_csv")
    for k in ("kernel", "op", "workload", "digest", "command", "out"):
        t.add_argument(f"--{k}", required=True)
    a = ap.parse_args(argv)
    if a.cmd == "stats":
        text = stats(a.csv, a.command)
    else:
        text = traffic(a.fetch_csv, a.write_csv, a.kernel, a.op, a.workload, a.digest, a.command)
    with open(a.out, "w") as f:
        f.write(text)
    sys.stdout.write(text)


if __name__ == "__main__":
    main()
