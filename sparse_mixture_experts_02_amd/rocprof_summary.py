"""Summaries of rocprofv3 CSV output (kernel statistics and per-dispatch counters).

    python -m sparse_mixture_experts_02_amd.rocprof_summary stats <dir>
    python -m sparse_mixture_experts_02_amd.rocprof_summary pmc <dir> [--calib-kernel NAME --calib-bytes N]
    python -m sparse_mixture_experts_02_amd.rocprof_summary mfma <dir>

`stats` reads the *_kernel_stats.csv that `rocprofv3 --kernel-trace --stats --output-format csv`
writes; `pmc` reads the *_counter_collection.csv of a `rocprofv3 --pmc ... --output-format csv`
run and prints each counter's mean per dispatch for every kernel. With a calibration kernel of
known traffic (an elementwise copy that reads and writes N bytes), FETCH_SIZE and WRITE_SIZE are
also given as a scale factor (known bytes / counted bytes) and as scaled bytes per dispatch.
`mfma` reads a `--pmc GRBM_GUI_ACTIVE SQ_VALU_MFMA_BUSY_CYCLES` run and prints, per kernel, the
mean dispatch duration, the effective clock (GRBM_GUI_ACTIVE is summed over the 8 XCDs) and the
fraction of SIMD cycles the matrix cores were busy (SQ_VALU_MFMA_BUSY_CYCLES over
GRBM_GUI_ACTIVE / 8 x 1024 SIMDs).
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob
import os
import sys


def _find(d: str, suffix: str) -> list:
    return sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True))


def kernel_stats(d: str) -> list:
    rows = []
    for path in _find(d, "kernel_stats.csv"):
        with open(path, newline="") as f:
            for r in csv.DictReader(f):
                rows.append({"name": r["Name"], "calls": int(r["Calls"]), "avg_us": float(r["AverageNs"]) / 1e3,
                             "min_us": float(r["MinNs"]) / 1e3, "max_us": float(r["MaxNs"]) / 1e3,
                             "pct": float(r["Percentage"])})
    return rows


def counters(d: str) -> dict:
    """{(kernel, counter): [values per dispatch]}"""
    out = collections.defaultdict(list)
    for path in _find(d, "counter_collection.csv"):
        with open(path, newline="") as f:
            for r in csv.DictReader(f):
                out[(r["Kernel_Name"], r["Counter_Name"])].append(float(r["Counter_Value"]))
    return out


def dispatches(d: str) -> dict:
    """{kernel: [{counter: value, ..., "dur_ns": duration} per dispatch]}"""
    per = collections.defaultdict(dict)
    for path in _find(d, "counter_collection.csv"):
        with open(path, newline="") as f:
            for r in csv.DictReader(f):
                key = (r["Kernel_Name"], r["Dispatch_Id"])
                per[key][r["Counter_Name"]] = per[key].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
                per[key]["dur_ns"] = float(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    out = collections.defaultdict(list)
    for (k, _), v in per.items():
        out[k].append(v)
    return out


XCDS, SIMDS = 8, 1024


def short(name: str, n: int = 70) -> str:
    return name if len(name) <= n else name[: n - 3] + "..."


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("mode", choices=["stats", "pmc", "mfma"])
    ap.add_argument("dir")
    ap.add_argument("--calib-kernel", default="AUnaryFunctor",
                    help="substring naming the calibration kernel (torch.mul by a scalar)")
    ap.add_argument("--calib-bytes", type=float, default=0.0)
    a = ap.parse_args(argv)
    if a.mode == "stats":
        rows = kernel_stats(a.dir)
        print(f"{'kernel':72s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s} {'pct':>6s}")
        for r in sorted(rows, key=lambda r: -r["pct"]):
            print(f"{short(r['name'], 72):72s} {r['calls']:6d} {r['avg_us']:10.2f} {r['min_us']:10.2f} "
                  f"{r['max_us']:10.2f} {r['pct']:6.2f}")
        return 0
    if a.mode == "mfma":
        print(f"{'kernel':72s} {'n':>4s} {'avg_us':>9s} {'clock_GHz':>9s} {'mfma_busy':>9s}")
        for k, ds in sorted(dispatches(a.dir).items()):
            ds = [x for x in ds if x.get("GRBM_GUI_ACTIVE", 0) > 0 and "SQ_VALU_MFMA_BUSY_CYCLES" in x]
            if not ds:
                continue
            gui = sum(x["GRBM_GUI_ACTIVE"] for x in ds)
            busy = sum(x["SQ_VALU_MFMA_BUSY_CYCLES"] for x in ds)
            dur = sum(x["dur_ns"] for x in ds)
            if busy <= 0:
                continue
            print(f"{short(k, 72):72s} {len(ds):4d} {dur / len(ds) / 1e3:9.2f} {gui / XCDS / dur:9.2f} "
                  f"{busy / (gui / XCDS * SIMDS):9.3f}")
        return 0
    c = counters(a.dir)
    scale = {}
    if a.calib_bytes > 0:
        for cname in ("FETCH_SIZE", "WRITE_SIZE"):
            vals = [v for (k, n), vs in c.items() if n == cname and a.calib_kernel in k for v in vs]
            if vals:
                counted = sum(vals) / len(vals) * 1024.0       # the counters are in KiB
                scale[cname] = a.calib_bytes / counted if counted > 0 else float("nan")
                print(f"calibration: {cname} reads {counted / 2**20:.1f} MiB for a kernel that moves "
                      f"{a.calib_bytes / 2**20:.1f} MiB -> scale {scale[cname]:.3f}")
    print(f"{'kernel':72s} {'counter':30s} {'n':>4s} {'mean':>14s} {'scaled_MiB':>11s}")
    for (k, n), vs in sorted(c.items()):
        mean = sum(vs) / len(vs)
        scaled = f"{mean * 1024.0 * scale[n] / 2**20:11.1f}" if n in scale else ""
        print(f"{short(k, 72):72s} {n:30s} {len(vs):4d} {mean:14.6g} {scaled}")
    return 0


if __name__ == "__main__":
    sys.exit(main())
