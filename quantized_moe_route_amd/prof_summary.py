"""Summaries of rocprofv3 output for the committed profiles.

  stats    kernel-trace statistics (the *_kernel_stats.csv of `rocprofv3 --stats`)
           -> a short text table;
  counters per-dispatch means of every counter in one or more `rocprofv3 --pmc` runs, per
           kernel family (given as name=regex pairs) -> a short text table;
  traffic  HBM bytes per launch of one kernel from two `rocprofv3 --pmc` runs
           (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch), each scaled by what the
           same counter reads for a copy kernel of known size run in the same process
           -> a JSON record that bench.py reports as roofline.traffic while the
           kernel's sources are unchanged (kernel_source_hash).
"""
from __future__ import annotations

import argparse
import csv
import json
import re
import statistics
import sys


def _rows(path):
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def kernel_stats(path: str, top: int = 12) -> str:
    rows = _rows(path)
    out = [f"{'kernel':60s} {'calls':>7s} {'avg us':>10s} {'min us':>10s} {'max us':>10s} {'share %':>8s}"]
    for r in rows[:top]:
        name = r["Name"]
        name = name if len(name) <= 60 else name[:57] + "..."
        out.append(f"{name:60s} {int(r['Calls']):7d} {float(r['AverageNs']) / 1e3:10.2f} "
                   f"{float(r['MinNs']) / 1e3:10.2f} {float(r['MaxNs']) / 1e3:10.2f} {float(r['Percentage']):8.2f}")
    return "\n".join(out)


def counter_avg(path: str, counter: str, name_re: str, min_value: float = 0.0):
    """Mean per-dispatch value of `counter` over dispatches whose kernel name matches
    (and whose value is at least min_value)."""
    vals = [float(r["Counter_Value"]) for r in _rows(path)
            if r["Counter_Name"] == counter and re.search(name_re, r["Kernel_Name"])]
    vals = [v for v in vals if v >= min_value]
    return (statistics.fmean(vals) if vals else None), len(vals)


def counter_table(paths, kernels) -> str:
    """Mean per-dispatch value of every counter found in the csv files, per kernel family
    (kernels: list of (name, regex)); SQ counters are totals over the device."""
    vals = {}
    for p in paths:
        for r in _rows(p):
            for name, rx in kernels:
                if re.search(rx, r["Kernel_Name"]):
                    vals.setdefault((r["Counter_Name"], name), []).append(float(r["Counter_Value"]))
    counters = sorted({c for c, _ in vals})
    names = [n for n, _ in kernels]
    out = [f"{'counter (mean per dispatch)':30s}" + "".join(f"{n:>18s}" for n in names)]
    for c in counters:
        row = f"{c:30s}"
        for n in names:
            v = vals.get((c, n))
            row += f"{statistics.fmean(v):18.4g}" if v else f"{'-':>18s}"
        out.append(row)
    return "\n".join(out)


def traffic(fetch_csv, write_csv, kernel_re, copy_re, copy_bytes):
    kf, nkf = counter_avg(fetch_csv, "FETCH_SIZE", kernel_re)
    kw, nkw = counter_avg(write_csv, "WRITE_SIZE", kernel_re)
    # the calibration copies are the copy dispatches whose counter reads at least 1/16 of
    # copy_bytes (smaller copies of the same kernel are the setup's uploads)
    floor = copy_bytes / 1024.0 / 16
    cf, ncf = counter_avg(fetch_csv, "FETCH_SIZE", copy_re, floor)
    cw, ncw = counter_avg(write_csv, "WRITE_SIZE", copy_re, floor)
    if None in (kf, kw, cf, cw) or cf == 0 or cw == 0:
        raise SystemExit(f"missing dispatches: kernel {nkf}/{nkw}, copy {ncf}/{ncw}")
    sf = copy_bytes / (cf * 1024.0)
    sw = copy_bytes / (cw * 1024.0)
    return {
        "fetch_kib_per_launch": kf, "write_kib_per_launch": kw, "launches": [nkf, nkw],
        "copy_bytes": copy_bytes, "copy_fetch_kib": cf, "copy_write_kib": cw,
        "fetch_scale": sf, "write_scale": sw,
        "hbm_read_bytes_per_launch": kf * 1024.0 * sf,
        "hbm_write_bytes_per_launch": kw * 1024.0 * sw,
        "hbm_bytes_per_launch": kf * 1024.0 * sf + kw * 1024.0 * sw,
    }


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    a = sub.add_parser("stats")
    a.add_argument("csv")
    a.add_argument("--top", type=int, default=12)
    c = sub.add_parser("counters")
    c.add_argument("csv", nargs="+")
    c.add_argument("--kernel", action="append", required=True, help="name=regex of a kernel family (repeatable)")
    b = sub.add_parser("traffic")
    b.add_argument("--fetch", required=True)
    b.add_argument("--write", required=True)
    b.add_argument("--kernel", required=True, help="regex of the kernel name")
    b.add_argument("--copy", default="direct_copy", help="regex of the calibration copy kernel")
    b.add_argument("--copy-bytes", type=int, required=True)
    b.add_argument("--hash", required=True, help="kernel_source_hash of the profiled sources")
    b.add_argument("--command", default="", help="the commands that produced the csv files")
    args = ap.parse_args(argv)
    if args.cmd == "stats":
        print(kernel_stats(args.csv, args.top))
        return
    if args.cmd == "counters":
        print(counter_table(args.csv, [tuple(k.split("=", 1)) for k in args.kernel]))
        return
    rec = traffic(args.fetch, args.write, args.kernel, args.copy, args.copy_bytes)
    rec["kernel_source_hash"] = args.hash
    rec["kernel"] = args.kernel
    rec["command"] = args.command
    json.dump(rec, sys.stdout, indent=1)
    print()


if __name__ == "__main__":
    main()
