"""Reduce rocprofv3 output to the figures the benchmark and its profile summaries use.

  python -m tiled_dense_gemm_major_amd.profsum trace DIR --kernel gemm_quad --timed 50
  python -m tiled_dense_gemm_major_amd.profsum traffic --kernel gemm_quad \\
      --fetch DIR --write DIR --copy-fetch DIR --copy-write DIR --copy-bytes 536870912 \\
      --workload "bf16 8192x8192x8192, B [N,K]" --out profiles/traffic_....json

`trace` reads the kernel trace (`--kernel-trace`) and prints the dispatch count and the
average, median, min and max duration of the named kernel, over all dispatches (or those
of `--range A:B`, in start order) and over the last `--timed` ones of them (the timed
region of a benchmark run).

`counters` reads counter runs (with their kernel traces) of the kernel and reports GPU
cycles per launch, the engine clock, MFMA utilisation and the LDS bank-conflict share.

`traffic` reads two counter runs of the kernel (`--pmc FETCH_SIZE`, `--pmc WRITE_SIZE`,
KiB per dispatch) and the same two counters for a plain device copy of `--copy-bytes`
bytes, scales each counter so that the copy reads and writes exactly its size, and
writes the per-launch HBM bytes with the digest of the kernel sources they belong to.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import statistics
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
# The sources that define the quad kernel for A [M,K], B [N,K], its compiled
# configurations and the table that picks one: counter figures taken on other sources
# are stale.  (The traffic record also stores the configuration it was taken on, which
# the benchmark compares with the table's current choice.)
KERNEL_SOURCES = [os.path.join(ROOT, "tiled_dense_gemm_major_amd", "csrc", f)
                  for f in ("kernels.hpp", "launch.hpp", "registry.hpp", "variants_quad.hip",
                            "tile_table.inc")]


def kernel_digest() -> str:
    """Digest of the kernel sources: counter figures taken on other sources are stale."""
    h = hashlib.sha256()
    for path in KERNEL_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _csv(directory: str, suffix: str):
    paths = sorted(glob.glob(os.path.join(directory, "**", "*" + suffix), recursive=True))
    if not paths:
        raise SystemExit(f"no *{suffix} under {directory}")
    rows = []
    for p in paths:
        with open(p, newline="") as f:
            rows += list(csv.DictReader(f))
    return rows


def _db_kernel_rows(directory: str):
    """Kernel dispatches from rocprofv3's SQLite output (*_results.db): name, start, end."""
    import sqlite3
    paths = sorted(glob.glob(os.path.join(directory, "**", "*_results.db"), recursive=True))
    rows = []
    for p in paths:
        db = sqlite3.connect(p)
        try:
            for name, start, end in db.execute("select name, start, end from kernels"):
                rows.append({"Kernel_Name": name, "Start_Timestamp": start,
                             "End_Timestamp": end})
        finally:
            db.close()
    return rows


def trace_durations_ns(directory: str, kernel: str):
    """Durations of the dispatches of the kernel whose name contains `kernel`, in order
    (from the CSV kernel trace, or else from the SQLite output)."""
    paths = glob.glob(os.path.join(directory, "**", "*kernel_trace.csv"), recursive=True)
    rows = _csv(directory, "kernel_trace.csv") if paths else _db_kernel_rows(directory)
    rows = [r for r in rows if kernel in r["Kernel_Name"]]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    return [int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in rows], \
        (rows[0]["Kernel_Name"] if rows else "")


def counter_per_dispatch(directory: str, kernel: str, counter: str):
    """Sum of `counter` over its instances, per dispatch of the matching kernel."""
    per = {}
    for r in _csv(directory, "counter_collection.csv"):
        if kernel in r["Kernel_Name"] and r["Counter_Name"] == counter:
            k = int(r["Dispatch_Id"])
            per[k] = per.get(k, 0.0) + float(r["Counter_Value"])
    if not per:
        raise SystemExit(f"no {counter} for {kernel!r} under {directory}")
    return [per[k] for k in sorted(per)]


def counter_instances(directory: str, kernel: str, counter: str):
    """Per dispatch of the matching kernel: (sum over the counter's instances, number of
    instances), in dispatch order."""
    per, n = {}, {}
    for r in _csv(directory, "counter_collection.csv"):
        if kernel in r["Kernel_Name"] and r["Counter_Name"] == counter:
            k = int(r["Dispatch_Id"])
            per[k] = per.get(k, 0.0) + float(r["Counter_Value"])
            n[k] = n.get(k, 0) + 1
    return [(per[k], n[k]) for k in sorted(per)]


def cmd_counters(args):
    """Counter runs of one kernel, joined with the kernel trace of the same runs: GPU
    cycles per launch (GRBM_GUI_ACTIVE over the XCDs it sums), the engine clock over the
    launch, MFMA
    utilisation (SQ_VALU_MFMA_BUSY_CYCLES over cycles x SIMDs) and the LDS bank-conflict
    share of LDS cycles (SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE), medians over the
    dispatches."""
    out = {"kernel": args.kernel}
    vals = {}
    for d in args.dirs:
        for c in ("GRBM_GUI_ACTIVE", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_LDS_BANK_CONFLICT",
                  "SQ_LDS_IDX_ACTIVE", "SQ_BUSY_CYCLES", "SQ_INSTS_LDS"):
            try:
                got = counter_instances(d, args.kernel, c)
            except SystemExit:
                continue
            if got:
                vals[c] = got
                out[c + "_median"] = statistics.median(v for v, _ in got)
                out[c + "_instances"] = got[0][1]
        if "GRBM_GUI_ACTIVE" in vals and "trace_us_median" not in out:
            try:
                dur, _ = trace_durations_ns(d, args.kernel)
            except SystemExit:
                dur = []
            if dur:
                out["trace_us_median"] = statistics.median(dur) / 1e3
                out["trace_dispatches"] = len(dur)
    if "GRBM_GUI_ACTIVE" in vals:
        g = statistics.median(v for v, _ in vals["GRBM_GUI_ACTIVE"])
        cycles = g / args.xcds                  # summed over the XCDs, each counting
        out["cycles_per_launch"] = cycles
        if "trace_us_median" in out:
            out["clock_mhz"] = cycles / out["trace_us_median"]
        if "SQ_VALU_MFMA_BUSY_CYCLES_median" in out:
            out["mfma_util"] = out["SQ_VALU_MFMA_BUSY_CYCLES_median"] / (cycles * args.simds)
    if "SQ_LDS_BANK_CONFLICT_median" in out and out.get("SQ_LDS_IDX_ACTIVE_median"):
        out["lds_bank_conflict_share"] = (out["SQ_LDS_BANK_CONFLICT_median"] /
                                          out["SQ_LDS_IDX_ACTIVE_median"])
    print(json.dumps(out, indent=1))


def cmd_trace(args):
    d, name = trace_durations_ns(args.dir, args.kernel)
    if not d:
        raise SystemExit(f"no dispatch of {args.kernel!r}")
    us = [x / 1e3 for x in d]
    if args.range:
        lo, hi = (int(x) for x in args.range.split(":"))
        us = us[lo:hi]
        if not us:
            raise SystemExit(f"no dispatch in range {args.range}")
    timed = us[-args.timed:] if args.timed else us
    out = {
        "kernel": name,
        "dispatches": len(us),
        "avg_us": statistics.fmean(us),
        "median_us": statistics.median(us),
        "min_us": min(us),
        "max_us": max(us),
        "timed": len(timed),
        "timed_avg_us": statistics.fmean(timed),
        "timed_median_us": statistics.median(timed),
    }
    print(json.dumps(out, indent=1))


def _table_choice(shape: str):
    """The library's configuration for "dtype,M,N,K,b_layout" (host-only query)."""
    from . import tgemm
    dt, m, n, k, lay = (int(x) for x in shape.split(","))
    return tgemm.query_config(dt, m, n, k, lay).as_dict()


def cmd_traffic(args):
    fetch = counter_per_dispatch(args.fetch, args.kernel, "FETCH_SIZE")
    write = counter_per_dispatch(args.write, args.kernel, "WRITE_SIZE")
    cfetch = counter_per_dispatch(args.copy_fetch, args.copy_kernel, "FETCH_SIZE")
    cwrite = counter_per_dispatch(args.copy_write, args.copy_kernel, "WRITE_SIZE")
    kib = args.copy_bytes / 1024.0
    fscale = kib / statistics.median(cfetch)
    wscale = kib / statistics.median(cwrite)
    # the first dispatch of a run may see cold caches and first-touch effects: the median
    fk, wk = statistics.median(fetch), statistics.median(write)
    fb, wb = fk * 1024 * fscale, wk * 1024 * wscale
    rec = {
        "kernel": args.kernel_name or args.kernel,
        "workload": args.workload,
        "kernel_digest": kernel_digest(),
        "tile_config": _table_choice(args.shape) if args.shape else None,
        "bytes_per_launch": fb + wb,
        "fetch_bytes_per_launch": fb,
        "write_bytes_per_launch": wb,
        "fetch_kib_raw": fk,
        "write_kib_raw": wk,
        "fetch_scale": fscale,
        "write_scale": wscale,
        "copy_fetch_kib_raw": statistics.median(cfetch),
        "copy_write_kib_raw": statistics.median(cwrite),
        "dispatches": [len(fetch), len(write)],
    }
    if args.out:
        with open(args.out, "w") as f:
            json.dump(rec, f, indent=1)
            f.write("\n")
    print(json.dumps(rec, indent=1))


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("trace")
    t.add_argument("dir")
    t.add_argument("--kernel", required=True)
    t.add_argument("--timed", type=int, default=0)
    t.add_argument("--range", default="",
                   help="A:B, only dispatches A..B-1 of the kernel (in start order)")
    k = sub.add_parser("counters")
    k.add_argument("dirs", nargs="+")
    k.add_argument("--kernel", required=True)
    k.add_argument("--simds", type=int, default=1024, help="SIMDs on the chip (256 CUs x 4)")
    k.add_argument("--xcds", type=int, default=8,
                   help="XCDs whose GRBM_GUI_ACTIVE the reported value sums")
    c = sub.add_parser("traffic")
    c.add_argument("--kernel", required=True)
    c.add_argument("--kernel-name", default="")
    c.add_argument("--fetch", required=True)
    c.add_argument("--write", required=True)
    c.add_argument("--copy-fetch", required=True)
    c.add_argument("--copy-write", required=True)
    c.add_argument("--copy-kernel", default="copyBuffer")
    c.add_argument("--copy-bytes", type=int, required=True)
    c.add_argument("--workload", default="")
    c.add_argument("--shape", default="",
                   help="dtype,M,N,K,b_layout of the product: its configuration is recorded")
    c.add_argument("--out", default="")
    args = ap.parse_args(argv)
    {"trace": cmd_trace, "traffic": cmd_traffic, "counters": cmd_counters}[args.cmd](args)


if __name__ == "__main__":
    sys.exit(main())
