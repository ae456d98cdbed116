"""Summaries of rocprofv3 CSV output (kernel statistics and per-dispatch counters).

    python -m sparse_mixture_experts_02_amd.rocprof_summary stats <dir>
    python -m sparse_mixture_experts_02_amd.rocprof_summary pmc <dir> [--calib-kernel NAME --calib-bytes N]
    python -m sparse_mixture_experts_02_amd.rocprof_summary mfma <dir>
    python -m sparse_mixture_experts_02_amd.rocprof_summary traffic <fetch_dir> <write_dir> --calib-bytes N

`stats` reads the *_kernel_stats.csv that `rocprofv3 --kernel-trace --stats --output-format csv`
writes; `pmc` reads the *_counter_collection.csv of a `rocprofv3 --pmc ... --output-format csv`
run and prints each counter's mean per dispatch for every kernel. With a calibration kernel of
known traffic (an elementwise copy that reads and writes N bytes), FETCH_SIZE and WRITE_SIZE are
also given as a scale factor (known bytes / counted bytes) and as scaled bytes per dispatch.
`mfma` reads a `--pmc GRBM_GUI_ACTIVE SQ_VALU_MFMA_BUSY_CYCLES` run and prints, per kernel, the
mean dispatch duration, the effective clock (GRBM_GUI_ACTIVE is summed over the 8 XCDs) and the
fraction of SIMD cycles the matrix cores were busy (SQ_VALU_MFMA_BUSY_CYCLES over
GRBM_GUI_ACTIVE / 8 x 1024 SIMDs).
`traffic` reads a FETCH_SIZE run and a WRITE_SIZE run (each with the calibration copy) and prints
the calibrated bytes per dispatch of the two grouped-GEMM launches (the SiLU one as gemm1_silu,
the other as gemm2) with a digest of the grouped-GEMM sources they measured, in the form
bench.py reads back.
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob
import hashlib
import os
import sys

CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")
GEMM_SOURCES = ("gemm.hip", "gemm_big.hip", "gemm_stream.hip")


def gemm_sources_digest() -> str:
    """sha256 over the grouped-GEMM kernel sources (traffic records name the code they measured)."""
    h = hashlib.sha256()
    for name in GEMM_SOURCES:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


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
    ap.add_argument("mode", choices=["stats", "pmc", "mfma", "traffic"])
    ap.add_argument("dir")
    ap.add_argument("write_dir", nargs="?", default=None, help="traffic mode: the WRITE_SIZE run")
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
    if a.mode == "traffic":
        return traffic(a)
    c = counters(a.dir)
    scale = {}
    if a.calib_bytes > 0:
        for cname in ("FETCH_SIZE", "WRITE_SIZE"):
            counted = _calib_counted(c, cname, a.calib_kernel)
            if counted is not None:
                scale[cname] = a.calib_bytes / counted if counted > 0 else float("nan")
                print(f"calibration: {cname} reads {counted / 2**20:.1f} MiB for a kernel that moves "
                      f"{a.calib_bytes / 2**20:.1f} MiB -> scale {scale[cname]:.3f}")
    print(f"{'kernel':72s} {'counter':30s} {'n':>4s} {'mean':>14s} {'scaled_MiB':>11s}")
    for (k, n), vs in sorted(c.items()):
        mean = sum(vs) / len(vs)
        scaled = f"{mean * 1024.0 * scale[n] / 2**20:11.1f}" if n in scale else ""
        print(f"{short(k, 72):72s} {n:30s} {len(vs):4d} {mean:14.6g} {scaled}")
    return 0


def _calib_counted(c: dict, cname: str, calib_kernel: str):
    """Bytes that counter `cname` reports for the calibration copy, or None if the run has none.
    The copy is the largest dispatch of its elementwise kernel: the program may launch the same
    kernel for smaller scalar multiplies of its own, which must not enter the scale."""
    vals = [v for (k, n), vs in c.items() if n == cname and calib_kernel in k for v in vs]
    return max(vals) * 1024.0 if vals else None   # the counters are in KiB


def _calibrated_means(d: str, cname: str, calib_kernel: str, calib_bytes: float) -> dict:
    c = counters(d)
    counted = _calib_counted(c, cname, calib_kernel)
    if counted is None:
        raise SystemExit(f"no calibration dispatch ({calib_kernel}) with {cname} in {d}")
    scale = calib_bytes / counted
    return {k: sum(vs) / len(vs) * 1024.0 * scale for (k, n), vs in c.items() if n == cname}, scale


def traffic(a) -> int:
    if not a.write_dir or a.calib_bytes <= 0:
        raise SystemExit("traffic mode needs <fetch_dir> <write_dir> --calib-bytes N")
    fetch, sf = _calibrated_means(a.dir, "FETCH_SIZE", a.calib_kernel, a.calib_bytes)
    write, sw = _calibrated_means(a.write_dir, "WRITE_SIZE", a.calib_kernel, a.calib_bytes)
    print(f"# calibration scale: FETCH_SIZE {sf:.3f}, WRITE_SIZE {sw:.3f}")
    print(f"# grouped GEMM sources sha256: {gemm_sources_digest()}")
    # the grouped GEMMs' first template argument is the SiLU flag (gemm_big_kernel<true, false>,
    # gemm_stream_kernel<true>, gemm_q4_kernel<true>)
    for label, flag in (("gemm1_silu", "<true"), ("gemm2", "<false")):
        ks = [k for k in fetch if "gemm" in k and "tail" not in k and flag in k]
        if len(ks) != 1:
            continue
        print(f"# {label} kernel: {ks[0]}")
        print(f"# {label} fetch_bytes: {int(round(fetch[ks[0]]))}")
        print(f"# {label} write_bytes: {int(round(write.get(ks[0], 0.0)))}")
    print(f"{'kernel':72s} {'fetch_MiB':>10s} {'write_MiB':>10s}")
    for k in sorted(fetch):
        print(f"{short(k, 72):72s} {fetch[k] / 2**20:10.1f} {write.get(k, 0.0) / 2**20:10.1f}")
    return 0


if __name__ == "__main__":
    sys.exit(main())
