"""Summaries of rocprofv3 output for the committed profiles.

    python3 profiling.py trace DIR [--match gemv]
        per-kernel calls and durations from a `--kernel-trace --stats` run

    python3 profiling.py traffic --fetch DIR --write DIR \\
        --copy-fetch DIR --copy-write DIR --copy-bytes N --key block_int4/m1 --out FILE
        HBM bytes per launch of the GEMV from FETCH_SIZE / WRITE_SIZE, each
        scaled by what the same counter reads for a plain copy of N bytes

    python3 profiling.py counters DIR --match gemm_kernel
        every counter of a `--pmc` run, per dispatch of the matching kernels
        (summed over the counter's instances: XCDs, SEs, channels)

Counters are taken per dispatch (rocprofv3 reports FETCH_SIZE and WRITE_SIZE
in KiB); the copy's dispatches are the largest ones of its run.
"""

from __future__ import annotations

import argparse
import collections
import csv
import glob
import json
import os
import sqlite3
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))


def _files(d: str, suffix: str):
    return sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True))


def _durations_db(d: str, match: str):
    """Kernel durations (ns) by name from rocprofv3's SQLite output."""
    out = collections.defaultdict(list)
    for f in _files(d, "_results.db"):
        con = sqlite3.connect(f)
        for name, dur in con.execute("select name, duration from kernels"):
            if match in name:
                out[name].append(float(dur))
    return out


def kernel_stats(d: str, match: str = ""):
    """(name, calls, avg, min, max, p10, p50, p90) in ns, from CSV or SQLite output."""
    rows = []
    for f in _files(d, "kernel_stats.csv"):
        for r in csv.DictReader(open(f)):
            if match in r["Name"]:
                rows.append((r["Name"], int(r["Calls"]), float(r["AverageNs"]), float(r["MinNs"]),
                             float(r["MaxNs"]), float("nan"), float("nan"), float("nan")))
    if not rows:
        for name, v in _durations_db(d, match).items():
            v = sorted(v)
            q = lambda p: v[min(len(v) - 1, int(p * len(v)))]
            rows.append((name, len(v), sum(v) / len(v), v[0], v[-1], q(0.1), q(0.5), q(0.9)))
    return rows


def counter_values(d: str, counter: str, match: str = ""):
    """Per-dispatch values of one counter for kernels whose name contains `match`."""
    per = collections.defaultdict(float)
    for f in _files(d, "counter_collection.csv"):
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] != counter or match not in r.get("Kernel_Name", ""):
                continue
            per[(f, r.get("Dispatch_Id", r.get("Correlation_Id", "")))] += float(r["Counter_Value"])
    for f in _files(d, "_results.db"):
        con = sqlite3.connect(f)
        q = "select dispatch_id, kernel_name, value from counters_collection where counter_name = ?"
        for disp, name, value in con.execute(q, (counter,)):
            if match in name:
                per[(f, disp)] += float(value)
    return list(per.values())


def _source_digest() -> str:
    sys.path.insert(0, ROOT)
    import bench
    return bench.source_digest()


def traffic(a) -> dict:
    def mean(v):
        if not v:
            raise SystemExit("no matching dispatches")
        return sum(v) / len(v)

    kib = 1024.0
    fetch = mean(counter_values(a.fetch, "FETCH_SIZE", a.match)) * kib
    write = mean(counter_values(a.write, "WRITE_SIZE", a.match)) * kib
    # the copy: its largest dispatches (the fill before it moves the same bytes once)
    cf = sorted(counter_values(a.copy_fetch, "FETCH_SIZE", ""))[-1] * kib
    cw = sorted(counter_values(a.copy_write, "WRITE_SIZE", ""))[-1] * kib
    kf, kw = a.copy_bytes / cf, a.copy_bytes / cw
    rec = {
        "source_digest": _source_digest(),
        "copy_bytes": a.copy_bytes,
        "copy_fetch_counter_bytes": cf,
        "copy_write_counter_bytes": cw,
        "fetch_scale": kf,
        "write_scale": kw,
        "per_launch_bytes": {
            a.key: {"fetch": round(fetch * kf), "write": round(write * kw), "total": round(fetch * kf + write * kw),
                    "fetch_counter_bytes": fetch, "write_counter_bytes": write},
        },
    }
    return rec


def counters(d: str, match: str):
    """{counter: (mean per dispatch, dispatches)} for kernels whose name contains `match`."""
    per = collections.defaultdict(lambda: collections.defaultdict(float))
    for f in _files(d, "_results.db"):
        con = sqlite3.connect(f)
        q = "select dispatch_id, kernel_name, counter_name, value from counters_collection"
        for disp, name, cname, value in con.execute(q):
            if match in name:
                per[cname][(f, disp)] += float(value)
    return {c: (sum(v.values()) / len(v), len(v)) for c, v in per.items()}


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("trace")
    t.add_argument("dir")
    t.add_argument("--match", default="")
    c = sub.add_parser("traffic")
    for k in ("fetch", "write", "copy_fetch", "copy_write"):
        c.add_argument("--" + k.replace("_", "-"), dest=k, required=True)
    c.add_argument("--copy-bytes", type=int, required=True)
    c.add_argument("--key", required=True)
    c.add_argument("--match", default="gemv")
    c.add_argument("--out", required=True)
    n = sub.add_parser("counters")
    n.add_argument("dir")
    n.add_argument("--match", default="")
    a = ap.parse_args(argv)
    if a.cmd == "trace":
        rows = kernel_stats(a.dir, a.match)
        if not rows:
            raise SystemExit("no matching kernels")
        print(f"{'kernel':64s} {'calls':>6s} {'avg us':>8s} {'min':>8s} {'p10':>8s} {'p50':>8s} {'p90':>8s} {'max':>8s}")
        for name, calls, avg, mn, mx, p10, p50, p90 in rows:
            print(f"{name[:64]:64s} {calls:6d} {avg / 1e3:8.3f} {mn / 1e3:8.3f} {p10 / 1e3:8.3f} {p50 / 1e3:8.3f} "
                  f"{p90 / 1e3:8.3f} {mx / 1e3:8.3f}")
    elif a.cmd == "counters":
        rows = counters(a.dir, a.match)
        if not rows:
            raise SystemExit("no matching dispatches")
        for c in sorted(rows):
            mean, n = rows[c]
            print(f"{c:32s} {mean:18.1f} per dispatch ({n} dispatches)")
    else:
        rec = traffic(a)
        with open(a.out, "w") as f:
            json.dump(rec, f, indent=1)
        json.dump(rec, sys.stdout, indent=1)
        print()


if __name__ == "__main__":
    main()
