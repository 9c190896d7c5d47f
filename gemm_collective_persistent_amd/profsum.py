"""Short text summaries of rocprofv3 output, for the ``profiles/`` folder.

Two summaries:

``stats``    per-kernel launch counts and durations from a
             ``--kernel-trace --stats`` run (``*_kernel_stats.csv``).
``traffic``  L2-to-fabric bytes per launch of one kernel from two ``--pmc``
             runs (FETCH_SIZE, then WRITE_SIZE; both in KiB per dispatch):
             what the XCDs' L2 caches fetch from and write to the memory
             fabric -- HBM, or the last-level (Infinity) cache, whose hits
             these counters cannot tell apart.  Each counter is scaled by what
             it reads for the three plain 1 GiB elementwise passes ``bench.py
             --copy-calibration`` makes (1 GiB read and 1 GiB written each, by
             construction), so the figure is in the same units as the
             algorithmic byte count.  The summary records the kernel-source
             digest it was taken on; ``bench.py`` ignores it once the kernels
             change.
``mfma``     matrix-core activity per launch of one kernel from one ``--pmc``
             run (SQ_VALU_MFMA_BUSY_CYCLES, SQ_INSTS_VALU_MFMA_MOPS_BF16,
             GRBM_GUI_ACTIVE) and the durations of a ``--kernel-trace`` run:
             the bf16 MFMA FLOPs the counters count (512 per MOP) against the
             algorithmic FLOPs, the clock (GPU-busy cycles over the
             duration), and the share of SIMD-cycles the matrix cores were
             busy.
``rates``    the communication-only launches of the unfused baselines
             (``bench.py --mode unfused``): L2-to-fabric bytes (FETCH_SIZE +
             WRITE_SIZE, calibrated as above) and durations per launch of one
             kernel, the launches of one call told apart by their order.

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
        f"# L2-to-fabric traffic of {op} on {workload} (rocprofv3 --pmc FETCH_SIZE, then WRITE_SIZE: bytes the "
        f"L2s fetch from and write to the memory fabric, HBM and last-level-cache hits alike)",
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


def _durations(trace_csv: str, kernel: str):
    rows = [r for r in csv.DictReader(open(trace_csv)) if kernel in r["Kernel_Name"]]
    rows.sort(key=lambda r: int(r["Dispatch_Id"]))
    return [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) for r in rows]


def mfma(pmc_csv: str, trace_csv: str, kernel: str, op: str, workload: str, flops: float, digest: str,
         command: str) -> str:
    def per(counter):
        return [float(r["Counter_Value"]) for r in _readings(pmc_csv, counter) if kernel in r["Kernel_Name"]]
    busy, mops, gui = per("SQ_VALU_MFMA_BUSY_CYCLES"), per("SQ_INSTS_VALU_MFMA_MOPS_BF16"), per("GRBM_GUI_ACTIVE")
    pdur = [int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in _readings(pmc_csv, "GRBM_GUI_ACTIVE")
            if kernel in r["Kernel_Name"]]
    dur = _durations(trace_csv, kernel)
    if not busy or not mops or not gui or not dur or not pdur:
        raise SystemExit(f"kernel {kernel!r} not found in both runs")
    b, m, g, d, pd = (statistics.median(x) for x in (busy, mops, gui, dur, pdur))
    # GRBM_GUI_ACTIVE counts GPU-busy cycles; summed over the 8 XCDs it reads
    # 8x the clock times the duration (the counter run's own duration)
    xcds = 8 if g / pd > 3.5 else 1
    clk_mhz = g / xcds / pd * 1e3
    simds = 256 * 4
    util = b / (g / xcds * simds)
    mflops = m * 512
    return "\n".join([
        f"# matrix-core activity of {op} on {workload} (rocprofv3 --pmc; durations from --kernel-trace)",
        f"command_pmc: {command.replace('PMC', 'SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_BF16 GRBM_GUI_ACTIVE')}",
        f"command_trace: {command.replace('--pmc PMC', '--kernel-trace')}",
        f"kernel: {kernel}",
        f"launches: {len(busy)} (pmc run), {len(dur)} (trace run); medians below",
        f"duration_us: {d / 1e3:.1f} (trace run); {pd / 1e3:.1f} (counter run)",
        f"grbm_gui_active_cycles: {g:.0f} (summed over {xcds} XCDs)",
        f"clock_mhz: {clk_mhz:.0f}",
        f"mfma_busy_simd_cycles: {b:.0f}",
        f"mfma_busy_fraction: {util:.4f}",
        f"mfma_bf16_flops_counted: {mflops:.4e}",
        f"algorithmic_flops: {flops:.4e}",
        f"counted_over_algorithmic: {mflops / flops:.4f}" if flops else "counted_over_algorithmic: n/a",
        f"tflops_at_duration: {mflops / (d * 1e-9) / 1e12:.1f}",
        f"source_digest: {digest}",
    ]) + "\n"


def rates(fetch_csv: str, write_csv: str, trace_csv: str, kernel: str, launches: int, which: int, label: str,
          nbytes: float, digest: str, command: str) -> str:
    fr, wr = _readings(fetch_csv, "FETCH_SIZE"), _readings(write_csv, "WRITE_SIZE")

    def calib(rows):
        big = [float(r["Counter_Value"]) * 1024 for r in rows if CALIB_KERNEL in r["Kernel_Name"]
               and float(r["Counter_Value"]) * 1024 > CALIB_BYTES / 8]
        if not big:
            raise SystemExit("no 1 GiB calibration copy found (run bench.py with --copy-calibration)")
        return CALIB_COPIES * CALIB_BYTES / sum(big)

    def pick(vals):
        return [v for i, v in enumerate(vals) if i % launches == which]
    fk = pick([float(r["Counter_Value"]) * 1024 for r in fr if kernel in r["Kernel_Name"]])
    wk = pick([float(r["Counter_Value"]) * 1024 for r in wr if kernel in r["Kernel_Name"]])
    dk = pick(_durations(trace_csv, kernel))
    if not fk or not wk or not dk:
        raise SystemExit(f"kernel {kernel!r} launch {which} of {launches} not found")
    f_b, w_b = statistics.median(fk) * calib(fr), statistics.median(wk) * calib(wr)
    d = statistics.median(dk)
    return "\n".join([
        f"# {label}: launch {which + 1} of the {launches} an unfused call makes",
        f"command_fetch: {command.replace('PMC', 'FETCH_SIZE')}",
        f"command_write: {command.replace('PMC', 'WRITE_SIZE')}",
        f"command_trace: {command.replace('--pmc PMC', '--kernel-trace')}",
        f"kernel: {kernel}",
        f"launches: {len(fk)} (fetch run), {len(wk)} (write run), {len(dk)} (trace run); medians below",
        f"duration_us: {d / 1e3:.1f}",
        f"l2_fabric_bytes: {f_b + w_b:.0f} (fetch {f_b:.0f}, write {w_b:.0f})",
        f"l2_fabric_gb_s: {(f_b + w_b) / (d * 1e-9) / 1e9:.1f}",
        f"algorithmic_bytes: {nbytes:.0f}",
        f"algorithmic_gb_s: {nbytes / (d * 1e-9) / 1e9:.1f}",
        f"fraction_of_hbm_peak_8tb_s: {nbytes / (d * 1e-9) / 8e12:.3f}",
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
    m = sub.add_parser("mfma")
    m.add_argument("pmc_csv")
    m.add_argument("trace_csv")
    for k in ("kernel", "op", "workload", "digest", "command", "out"):
        m.add_argument(f"--{k}", required=True)
    m.add_argument("--flops", type=float, required=True)
    r = sub.add_parser("rates")
    r.add_argument("fetch_csv")
    r.add_argument("write_csv")
    r.add_argument("trace_csv")
    for k in ("kernel", "label", "digest", "command", "out"):
        r.add_argument(f"--{k}", required=True)
    r.add_argument("--launches", type=int, required=True)
    r.add_argument("--which", type=int, required=True)
    r.add_argument("--bytes", type=float, required=True)
    a = ap.parse_args(argv)
    if a.cmd == "stats":
        text = stats(a.csv, a.command)
    elif a.cmd == "traffic":
        text = traffic(a.fetch_csv, a.write_csv, a.kernel, a.op, a.workload, a.digest, a.command)
    elif a.cmd == "mfma":
        text = mfma(a.pmc_csv, a.trace_csv, a.kernel, a.op, a.workload, a.flops, a.digest, a.command)
    else:
        text = rates(a.fetch_csv, a.write_csv, a.trace_csv, a.kernel, a.launches, a.which, a.label, a.bytes,
                     a.digest, a.command)
    with open(a.out, "w") as f:
        f.write(text)
    sys.stdout.write(text)


if __name__ == "__main__":
    main()
