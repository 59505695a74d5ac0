#!/usr/bin/env python3
"""Turn rocprofv3 output of bench.py runs into the short summaries kept under profiles/.

  python bench_profiles.py stats --csv <kernel_stats.csv> --bench <bench stdout> --cmd "<command>"
                                 --out profiles/<kernel>_<workload>_kernel_stats.txt
  python bench_profiles.py pmc --kernel k_partial_mfma --workload v3-b1 --fetch <csv> --write <csv>
                               --cal-fetch <csv> --cal-write <csv> --cal-bytes N --cmd "<commands>"
  python bench_profiles.py sq --kernel k_partial_mfma --workload v3-b64-var --csv <csv> [<csv> ...]
                              --cmd "<commands>" [--tiles-per-wg T]
  python bench_profiles.py ceiling --csv <kernel_stats.csv> --trace <kernel_trace.csv> --bench <stdout>
                                   --cmd "<command>" --out profiles/<name>.txt

The sq form averages per dispatch every SQ / GRBM counter (and the derived MfmaUtil) found for one
kernel in the given counter runs and writes profiles/<kernel>_<workload>_sq.txt: instructions per
wave by class and the MFMA busy share.  The ceiling form summarises a --copy-calibration run: the
copy and read-only reduction kernels and their bandwidths.

The pmc form reads per-dispatch FETCH_SIZE and WRITE_SIZE (KiB) of one kernel from two separate
counter runs, scales each by what the same counter reads for a plain device copy of known size
(copy kernels read and write exactly N bytes), and writes profiles/<kernel>_<workload>_pmc.json
(HBM bytes per launch, keyed to the kernel source it was measured on) plus a .txt summary.
"""
from __future__ import annotations

import argparse
import csv
import json
import os
import statistics
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)


def _rows(path):
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _col(row, *names):
    for n in names:
        if n in row:
            return row[n]
    raise KeyError(f"none of {names} in {list(row)}")


def counter_per_dispatch(path, counter, kernel_substr):
    """Mean counter value over the dispatches whose kernel name contains kernel_substr."""
    vals = {}
    for r in _rows(path):
        if _col(r, "Counter_Name", "counter_name") != counter:
            continue
        if kernel_substr not in _col(r, "Kernel_Name", "kernel_name"):
            continue
        d = _col(r, "Dispatch_Id", "dispatch_id")
        vals[d] = vals.get(d, 0.0) + float(_col(r, "Counter_Value", "counter_value"))
    if not vals:
        raise SystemExit(f"{path}: no {counter} rows for kernels matching {kernel_substr!r}")
    return statistics.mean(vals.values()), len(vals)


def cmd_stats(a):
    rows = _rows(a.csv)
    bench = None
    with open(a.bench) as f:
        for line in f:
            line = line.strip()
            if line.startswith("{") and '"metric"' in line:
                bench = json.loads(line)
    lines = [f"# rocprofv3 kernel-trace summary: {a.title}", "", "Command:", "", "    " + a.cmd, "",
             "| kernel | calls | avg us | min us | max us | share % |", "|---|---|---|---|---|---|"]
    for r in rows:
        name = _col(r, "Name", "KernelName", "Kernel_Name")
        if name.startswith("__amd") or "elementwise" in name or "spin_kernel" in name or "fill" in name:
            continue
        short = name.split("(")[0].replace("void ", "")
        lines.append(f"| {short} | {_col(r, 'Calls')} | {float(_col(r, 'AverageNs')) / 1e3:.2f} | "
                     f"{float(_col(r, 'MinNs')) / 1e3:.2f} | {float(_col(r, 'MaxNs')) / 1e3:.2f} | "
                     f"{float(_col(r, 'Percentage')):.1f} |")
    if a.trace and a.by_grid:
        # one kernel serves several shapes: split its dispatches by launch grid
        grp = {}
        for r in _rows(a.trace):
            name = _col(r, "Kernel_Name").split("(")[0].replace("void ", "")
            if not name.startswith("mla::"):
                continue
            grid = "x".join(str(int(_col(r, f"Grid_Size_{d}")) // max(1, int(_col(r, f"Workgroup_Size_{d}"))))
                            for d in "XYZ")
            grp.setdefault((name, grid), []).append(
                (int(_col(r, "End_Timestamp")) - int(_col(r, "Start_Timestamp"))) / 1e3)
        lines += ["", "Dispatches by launch grid (workgroups x, y, z):", "",
                  "| kernel | grid | calls | avg us | median us |", "|---|---|---|---|---|"]
        for (name, grid), v in grp.items():
            lines.append(f"| {name} | {grid} | {len(v)} | {statistics.mean(v):.2f} | {statistics.median(v):.2f} |")
    if a.trace and bench and not a.by_grid:
        # dispatch order in a bench.py run: the steps (warm-up, graph replays, spread replays), then
        # kernel_reps back-to-back launches of each kernel, then (--kernel-in-step) kernel_reps whole
        # steps with an event pair around each call
        in_step = "kernels_us_in_step" in bench
        disp = {}
        for r in _rows(a.trace):
            name = _col(r, "Kernel_Name").split("(")[0].replace("void ", "")
            disp.setdefault(name, []).append((int(_col(r, "Start_Timestamp")), int(_col(r, "End_Timestamp"))))
        L = a.loop
        mean_us = lambda v: f"{statistics.mean(e - s_ for s_, e in v) / 1e3:.2f}" if v else "-"
        lines += ["", "Average duration per launch (us) by part of the run: the steps (graph replays and warm-up), "
                      f"the bench's {L} back-to-back launches of the kernel alone" +
                      (f", and its {L} whole steps with an event pair per call" if in_step else "") + ":", "",
                  "| kernel | steps | back to back |" + (" in steps, events |" if in_step else ""),
                  "|---|---|---|" + ("---|" if in_step else "")]
        for name, v in disp.items():
            if not name.startswith("mla::"):
                continue
            v.sort()
            if in_step:
                steps, b2b, ins = v[:-2 * L], v[-2 * L:-L], v[-L:]
                lines.append(f"| {name} | {mean_us(steps)} | {mean_us(b2b)} | {mean_us(ins)} |")
            else:
                steps, b2b = v[:-L], v[-L:]
                lines.append(f"| {name} | {mean_us(steps)} | {mean_us(b2b)} |")
    if bench:
        if "kernels_us" in bench:
            lines += ["", "bench.py line of the same run (HIP-event averages, us; back to back): " +
                      json.dumps(bench["kernels_us"])]
            if "kernels_us_in_step" in bench:
                lines += ["bench.py, in whole steps with an event pair per call (us): " +
                          json.dumps(bench["kernels_us_in_step"])]
        else:
            lines += ["", "bench.py line of the same run:"]
        lines += [f"ms_per_step {bench['ms_per_step']}, value {bench['value']} {bench['unit']}, "
                  f"roofline {json.dumps(bench['roofline'])}"]
    with open(a.out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def cmd_pmc(a):
    from bench import KERNEL_SOURCES, source_hash
    fetch_kib, n1 = counter_per_dispatch(a.fetch, "FETCH_SIZE", a.kernel)
    write_kib, n2 = counter_per_dispatch(a.write, "WRITE_SIZE", a.kernel)
    cal_f, _ = counter_per_dispatch(a.cal_fetch, "FETCH_SIZE", a.cal_kernel)
    cal_w, _ = counter_per_dispatch(a.cal_write, "WRITE_SIZE", a.cal_kernel)
    kf = a.cal_bytes / (cal_f * 1024.0)     # true bytes per counted byte, reads
    kw = a.cal_bytes / (cal_w * 1024.0)     # same, writes
    fetch_b = fetch_kib * 1024.0 * kf
    write_b = write_kib * 1024.0 * kw
    out = {"kernel": a.kernel, "workload": a.workload, "source_hash": source_hash(KERNEL_SOURCES[a.kernel]),
           "fetch_kib_per_dispatch": fetch_kib, "write_kib_per_dispatch": write_kib,
           "dispatches": [n1, n2], "copy_scale_fetch": kf, "copy_scale_write": kw,
           "hbm_bytes_per_launch": round(fetch_b + write_b), "hbm_read_bytes": round(fetch_b),
           "hbm_write_bytes": round(write_b), "commands": a.cmd}
    base = os.path.join(ROOT, "profiles", f"{a.kernel}_{a.workload}_pmc")
    with open(base + ".json", "w") as f:
        json.dump(out, f, indent=1)
    txt = [f"# rocprofv3 counters: {a.kernel} on {a.workload}", "", "Commands:", ""]
    txt += ["    " + c for c in a.cmd.split(" ;; ")]
    txt += ["", f"FETCH_SIZE {fetch_kib:.1f} KiB/dispatch ({n1} dispatches), WRITE_SIZE {write_kib:.1f} KiB/dispatch "
                f"({n2} dispatches)",
            f"copy calibration ({a.cal_bytes} B read + written by {a.cal_kernel}): FETCH_SIZE scale {kf:.4f}, "
            f"WRITE_SIZE scale {kw:.4f}",
            f"HBM bytes per launch: read {fetch_b:.0f}, write {write_b:.0f}, total {fetch_b + write_b:.0f}"]
    with open(base + ".txt", "w") as f:
        f.write("\n".join(txt) + "\n")
    print("\n".join(txt))


def cmd_sq(a):
    vals = {}   # counter -> {dispatch: value}
    for path in a.csv:
        for r in _rows(path):
            if a.kernel not in _col(r, "Kernel_Name", "kernel_name"):
                continue
            c = _col(r, "Counter_Name", "counter_name")
            d = (path, _col(r, "Dispatch_Id", "dispatch_id"))
            vals.setdefault(c, {}).setdefault(d, 0.0)
            vals[c][d] += float(_col(r, "Counter_Value", "counter_value"))
    if not vals:
        raise SystemExit(f"no counter rows for kernels matching {a.kernel!r}")
    mean = {c: statistics.mean(v.values()) for c, v in vals.items()}
    n = {c: len(v) for c, v in vals.items()}
    waves = mean.get("SQ_WAVES")
    txt = [f"# rocprofv3 SQ counters: {a.kernel} on {a.workload}", "", "Commands:", ""]
    txt += ["    " + c for c in a.cmd.split(" ;; ")]
    txt += ["", "| counter | per dispatch | per wave | dispatches |", "|---|---|---|---|"]
    for c in sorted(mean):
        pw = f"{mean[c] / waves:.1f}" if waves and c.startswith("SQ_INSTS") else ""
        txt.append(f"| {c} | {mean[c]:.6g} | {pw} | {n[c]} |")
    if waves and a.tiles_per_wg:
        txt += ["", f"Per 32-token tile and wave ({a.tiles_per_wg} tiles per workgroup):"]
        for c in ("SQ_INSTS_MFMA", "SQ_INSTS_VALU", "SQ_INSTS_SALU", "SQ_INSTS_LDS"):
            if c in mean:
                txt.append(f"    {c}: {mean[c] / waves / a.tiles_per_wg:.1f}")
    if "MfmaUtil" in mean:
        txt += ["", f"MFMA busy (MfmaUtil: SQ_VALU_MFMA_BUSY_CYCLES over GRBM_GUI_ACTIVE x SIMDs): "
                    f"{mean['MfmaUtil']:.2f} %"]
    out = os.path.join(ROOT, "profiles", f"{a.kernel}_{a.workload}_sq.txt")
    with open(out, "w") as f:
        f.write("\n".join(txt) + "\n")
    print("\n".join(txt))


def cmd_ceiling(a):
    rows = _rows(a.csv)
    meas = None
    with open(a.bench) as f:
        for line in f:
            if line.startswith("{") and "copy_calibration_bytes" in line:
                meas = json.loads(line)
    txt = [f"# HBM streaming ceiling on this part: plain device copy and read-only reduction", "", "Command:", "",
           "    " + a.cmd, "", "| kernel | calls | avg us | min us |", "|---|---|---|---|"]
    for r in rows:
        name = _col(r, "Name", "KernelName", "Kernel_Name").split("(")[0].replace("void ", "")
        txt.append(f"| {name[:90]} | {_col(r, 'Calls')} | {float(_col(r, 'AverageNs')) / 1e3:.2f} | "
                   f"{float(_col(r, 'MinNs')) / 1e3:.2f} |")
    if meas:
        txt += ["", "HIP-event measurement of the same run: " + json.dumps(meas)]
    with open(a.out, "w") as f:
        f.write("\n".join(txt) + "\n")
    print("\n".join(txt))


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="what", required=True)
    s = sub.add_parser("stats")
    s.add_argument("--csv", required=True)
    s.add_argument("--bench", required=True)
    s.add_argument("--cmd", required=True)
    s.add_argument("--title", default="")
    s.add_argument("--out", required=True)
    s.add_argument("--trace", default=None, help="kernel_trace.csv of the same run")
    s.add_argument("--loop", type=int, default=50, help="dispatches per kernel in the bench's timing loop")
    s.add_argument("--by-grid", action="store_true", help="split each kernel's dispatches by launch grid")
    p = sub.add_parser("pmc")
    p.add_argument("--kernel", required=True)
    p.add_argument("--workload", required=True)
    p.add_argument("--fetch", required=True)
    p.add_argument("--write", required=True)
    p.add_argument("--cal-fetch", required=True)
    p.add_argument("--cal-write", required=True)
    p.add_argument("--cal-bytes", type=int, required=True)
    p.add_argument("--cal-kernel", default="copy")
    p.add_argument("--cmd", required=True)
    q = sub.add_parser("sq")
    q.add_argument("--kernel", required=True)
    q.add_argument("--workload", required=True)
    q.add_argument("--csv", nargs="+", required=True)
    q.add_argument("--cmd", required=True)
    q.add_argument("--tiles-per-wg", type=float, default=0.0)
    c = sub.add_parser("ceiling")
    c.add_argument("--csv", required=True)
    c.add_argument("--bench", required=True)
    c.add_argument("--cmd", required=True)
    c.add_argument("--out", required=True)
    a = ap.parse_args()
    {"stats": cmd_stats, "pmc": cmd_pmc, "sq": cmd_sq, "ceiling": cmd_ceiling}[a.what](a)


if __name__ == "__main__":
    main()
