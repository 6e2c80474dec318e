#!/usr/bin/env python3
"""Benchmark of libtgemm's hot path: one step = one C = A x B^T product of the headline
workload (bf16, M = N = K = 8192, A [M,K] and B [N,K] K-major, inputs uniform[-1,1]
rounded to bf16 from SplitMix64 seed 3, fp32 sums, bf16 output), inputs resident in HBM.

Prints ONE JSON line (stdout).  Progress goes to stderr.

  python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--procs 3] [--no-cpu-baseline]

Protocol ("0. A Minimal Hopper Matmul", sections "Launch, verify, and benchmark" and
"Performance": verify once, then time repeated launches; the figure is the median of
three fresh processes):
  * the parent process generates the inputs once (CPU only; it never touches the GPU)
    and runs ``procs`` fresh child processes one after the other;
  * each child copies the inputs to the GPU, launches the product once, and then times
    exactly ``steps`` back-to-back launches after ``warmup`` untimed ones, with HIP events
    recorded on the launch stream (one pair around all of them, one pair around each)
    and device synchronisation on both sides; two clock stamps around the timed region
    give the engine clock each XCD held meanwhile (reported as their mean);
  * the first child also checks its first result against the CPU oracle on the leading
    rows of C (every column, the full K) before it times anything, and times that oracle
    run as the CPU baseline; a mismatch ends the benchmark with an error;
  * ``value`` is the median process's whole-region rate; ``roofline.achieved`` is the
    algorithmic FLOP of one launch over that process's mean per-launch event time.
With --procs 1 the measurement runs in the bench process itself (the form to run under a
profiler).
"""
from __future__ import annotations

import argparse
import json
import os
import subprocess
import sys
import tempfile
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from tiled_dense_gemm_major_amd import roofline  # noqa: E402
from tiled_dense_gemm_major_amd.profsum import kernel_digest  # noqa: E402
from tiled_dense_gemm_major_amd.inputs import BF16, WORKLOADS  # noqa: E402

HEADLINE = "bf16_8192"
METRIC = "GEMM TFLOP/s at 8192^3 bf16 K-major (1 MI355X) and % of MFMA peak"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gemm_quad_bf16_8192.json")
CHILD_TAG = "BENCH_CHILD_RESULT "


def log(msg: str):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def measured_traffic(tile_config):
    """HBM bytes per launch from the committed rocprofv3 counter runs, or None when the
    kernel sources changed since they were taken or the table now picks another
    configuration."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_digest") != kernel_digest() or rec.get("tile_config") != tile_config:
        return None
    return rec.get("bytes_per_launch")


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def parity_and_cpu_baseline(A, B, C_gpu, w, budget_s: float):
    """The oracle (as it is) on the leading rows of C, sized to about budget_s seconds of
    host time: timed as the CPU baseline, and compared element by element with the same
    rows of the GPU's result."""
    import oracle
    threads = oracle.max_threads()
    probe_rows = 64
    t0 = time.perf_counter()
    oracle.gemm_rows(w.dtype, A, B, w.b_layout, 0, probe_rows)
    t_probe = time.perf_counter() - t0
    rows = int(max(probe_rows, min(w.M, probe_rows * budget_s / max(t_probe, 1e-3))))
    log(f"oracle: {probe_rows} rows took {t_probe:.2f}s; timing and checking {rows} rows on "
        f"{threads} threads")
    t0 = time.perf_counter()
    want = oracle.gemm_rows(w.dtype, A, B, w.b_layout, 0, rows)
    dt = time.perf_counter() - t0
    res = oracle.compare(w.dtype, w.K, C_gpu[:rows], want)
    flops = roofline.gemm_flops(rows, w.N, w.K)
    baseline = {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"rows 0..{rows - 1} of C ({rows}x{w.N} outputs, full K={w.K}) of the "
                   f"{w.describe()} product; {dt:.1f} s including decode and rounding"),
        "cpu_model": cpu_model(),
        "logical_cpus": os.cpu_count(),
    }
    parity = {"rows_checked": rows, "elements": res["n"], "n_fail": res["n_fail"],
              "max_err": res["max_err"], "max_err_over_tol": res["max_err_over_tol"],
              "rule": "|gpu - oracle| <= 1e-3*sqrt(K) + ulp(|oracle|), finite"}
    return baseline, parity


def engine_clock(before, after, wall_hz: float):
    """The engine clock from two clock stamps ([slot] = (engine cycles, wall ticks), a
    slot with no stamp holds zeros): for each compute unit stamped both times, its engine
    cycles over the wall time between the stamps, in MHz.  Returns (the median over the
    compute units, [min, p10, p90, max, count]), or (None, None) with no such unit."""
    per_cu = sorted((b[0] - a[0]) / (b[1] - a[1]) * wall_hz / 1e6
                    for a, b in zip(before, after) if a[1] > 0 and b[1] > a[1])
    if not per_cu:
        return None, None
    n = len(per_cu)
    return per_cu[n // 2], [per_cu[0], per_cu[n // 10], per_cu[-1 - n // 10], per_cu[-1], n]


def measure(args, A_bits, B_bits, verify: bool) -> dict:
    """Upload, verify (when asked), time; in the calling process."""
    import numpy as np
    import torch
    from tiled_dense_gemm_major_amd import tgemm

    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        sys.exit(1)
    tgemm.load()
    w = WORKLOADS[args.workload]
    tdt = torch.bfloat16 if w.dtype == BF16 else torch.float16
    A = torch.from_numpy(A_bits.view(np.int16)).cuda().view(tdt)
    B = torch.from_numpy(B_bits.view(np.int16)).cuda().view(tdt)
    C = torch.full((w.M, w.N), 0x7FC0 if w.dtype == BF16 else 0x7E00, dtype=torch.int16,
                   device="cuda").view(tdt)
    stream = torch.cuda.current_stream()

    def step():
        tgemm.gemm_ex(w.dtype, w.M, w.N, w.K, A, B, C, w.b_layout, None, stream)

    step()
    torch.cuda.synchronize()
    out = {}
    if verify:
        C_host = C.view(torch.int16).cpu().numpy().view(np.uint16)
        out["cpu_baseline"], out["parity"] = parity_and_cpu_baseline(
            A_bits, B_bits, C_host, w, args.cpu_budget_s)
        p = out["parity"]
        log(f"parity: {p['elements']} elements of rows 0..{p['rows_checked'] - 1}, "
            f"{p['n_fail']} failures, max err {p['max_err']:.3g} "
            f"({p['max_err_over_tol']:.3f} of tolerance)")

    for _ in range(args.warmup):
        step()
    stamps = torch.zeros((2, tgemm.CLOCK_STAMP_SLOTS, 2), dtype=torch.int64, device="cuda")
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    per = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    tgemm.clock_stamp(stamps[0], stream)
    start.record(stream)
    for ev0, ev1 in per:
        ev0.record(stream)
        step()
        ev1.record(stream)
    stop.record(stream)
    tgemm.clock_stamp(stamps[1], stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    per_ms = [a.elapsed_time(b) for a, b in per]
    st = stamps.cpu().tolist()
    clock_mhz, clock_spread = engine_clock(st[0], st[1], tgemm.wall_clock_hz())
    out.update({
        "total_ms": total_ms,
        "per_launch_ms": per_ms,
        "clock_mhz": clock_mhz,
        "clock_spread": clock_spread,
        "tile_config": tgemm.query_config(w.dtype, w.M, w.N, w.K, w.b_layout).as_dict(),
        "device": torch.cuda.get_device_name(0),
    })
    return out


def child(args):
    """One fresh process started by the parent: the inputs come from its files."""
    import numpy as np
    A_bits = np.load(os.path.join(args.inputs, "A.npy"))
    B_bits = np.load(os.path.join(args.inputs, "B.npy"))
    out = measure(args, A_bits, B_bits, args.verify)
    print(CHILD_TAG + json.dumps(out), flush=True)


def run_children(args, inputs_dir: str):
    results = []
    for i in range(args.procs):
        cmd = [sys.executable, os.path.abspath(__file__), "--child", "--inputs", inputs_dir,
               "--workload", args.workload, "--steps", str(args.steps),
               "--warmup", str(args.warmup), "--cpu-budget-s", str(args.cpu_budget_s)]
        if i == 0 and not args.no_cpu_baseline:
            cmd.append("--verify")
        log(f"process {i + 1} of {args.procs}")
        proc = subprocess.run(cmd, stdout=subprocess.PIPE, text=True)
        if proc.returncode != 0:
            log(f"process {i + 1} failed with exit status {proc.returncode}")
            sys.exit(proc.returncode if proc.returncode > 0 else 1)
        lines = [ln for ln in proc.stdout.splitlines() if ln.startswith(CHILD_TAG)]
        if not lines:
            log(f"process {i + 1} printed no result")
            sys.exit(1)
        r = json.loads(lines[-1][len(CHILD_TAG):])
        ms = r["total_ms"] / args.steps
        sp = r.get("clock_spread")
        spread = (f" (compute units: min {sp[0]:.0f}, p10 {sp[1]:.0f}, p90 {sp[2]:.0f}, "
                  f"max {sp[3]:.0f} MHz over {sp[4]})" if sp else "")
        log(f"process {i + 1}: {ms * 1e3:.1f} us/step, engine clock "
            f"{r['clock_mhz'] or 0:.0f} MHz over the timed region{spread}")
        results.append(r)
    return results


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--procs", type=int, default=3,
                    help="fresh processes to time; the reported figure is their median "
                         "(1: measure in this process)")
    ap.add_argument("--workload", default=HEADLINE, choices=list(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the oracle leg (and with it the parity check)")
    ap.add_argument("--cpu-budget-s", type=float, default=15.0)
    ap.add_argument("--child", action="store_true", help=argparse.SUPPRESS)
    ap.add_argument("--verify", action="store_true", help=argparse.SUPPRESS)
    ap.add_argument("--inputs", help=argparse.SUPPRESS)
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the product "
              f"is a single-device kernel library and no multi-GPU path is built.",
              file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0 or args.procs < 1:
        print("need --steps >= 1, --warmup >= 0, --procs >= 1", file=sys.stderr)
        sys.exit(2)
    if args.child:
        child(args)
        return

    import numpy as np
    w = WORKLOADS[args.workload]
    log(f"workload {w.describe()}")
    A_bits, B_bits = w.generate()
    if args.procs == 1:
        # one process: measure here (no child process; also the form to run under a
        # profiler, which starts the GPU before the program runs)
        results = [measure(args, A_bits, B_bits, not args.no_cpu_baseline)]
        report(args, w, results)
        return
    tmp = tempfile.mkdtemp(prefix="tgemm_bench_", dir="/dev/shm" if os.path.isdir("/dev/shm")
                           else None)
    try:
        np.save(os.path.join(tmp, "A.npy"), A_bits)
        np.save(os.path.join(tmp, "B.npy"), B_bits)
        del A_bits, B_bits
        results = run_children(args, tmp)
    finally:
        for f in ("A.npy", "B.npy"):
            try:
                os.remove(os.path.join(tmp, f))
            except OSError:
                pass
        os.rmdir(tmp)
    report(args, w, results)


def report(args, w, results):
    """The JSON line from the processes' measurements (the first one verified)."""
    first = results[0]
    if "parity" in first and first["parity"]["n_fail"]:
        log(f"parity failure: {first['parity']}")
        sys.exit(1)

    flops = roofline.gemm_flops(w.M, w.N, w.K)
    dname = "bf16" if w.dtype == BF16 else "f16"
    peak_tflops = roofline.PEAK_FLOPS[dname] / 1e12
    rates = [flops / (r["total_ms"] / args.steps * 1e-3) / 1e12 for r in results]
    order = sorted(range(len(results)), key=lambda i: rates[i])
    med = order[len(order) // 2]
    r = results[med]
    ms_per_step = r["total_ms"] / args.steps
    tflops = rates[med]
    launch_ms = sum(r["per_launch_ms"]) / len(r["per_launch_ms"])
    bound = roofline.bound(w.M, w.N, w.K, dname)
    if bound == "mfma":
        achieved = flops / (launch_ms * 1e-3) / 1e12
        peak, unit = peak_tflops, "TFLOP/s"
    else:
        achieved = roofline.compulsory_bytes(w.M, w.N, w.K) / (launch_ms * 1e-3) / 1e9
        peak, unit = roofline.HBM_BYTES_PER_S / 1e9, "GB/s"
    per_sorted = sorted(r["per_launch_ms"])
    log(f"median of {len(results)} processes: {ms_per_step * 1e3:.1f} us/step, "
        f"{tflops:.1f} TFLOP/s ({tflops / peak_tflops:.3f} of peak); per process "
        + ", ".join(f"{x:.1f}" for x in rates))

    out = {
        "metric": METRIC,
        "value": tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dname,
        "data": "synthetic",
        "config": {
            "workload": w.describe() + (" C=A*B^T" if w.b_layout == 0 else " C=A*B"),
            "M": w.M, "N": w.N, "K": w.K,
            "b_layout": "NK" if w.b_layout == 0 else "KN",
            "tile_config": r["tile_config"],
            "device": r["device"],
            "processes": len(results),
            "value_basis": "median process: 2MNK*steps over the HIP-event time of all "
                           "timed launches",
            "tflops_per_process": rates,
            "engine_clock_mhz_per_process": [x["clock_mhz"] for x in results],
            "engine_clock_mhz": r["clock_mhz"],
            "engine_clock_basis": "median over the compute units stamped before and after "
                                  "the timed region: engine cycles over wall time",
            "engine_clock_spread_mhz": dict(zip(("min", "p10", "p90", "max", "units"),
                                                r["clock_spread"])) if r.get("clock_spread")
            else None,
            "median_launch_ms": per_sorted[len(per_sorted) // 2],
            "p10_launch_ms": per_sorted[len(per_sorted) // 10],
            "p90_launch_ms": per_sorted[min(len(per_sorted) - 1, (9 * len(per_sorted)) // 10)],
            "avg_launch_ms": launch_ms,
            "frac_of_mfma_peak": tflops / peak_tflops,
            "parity": first.get("parity"),
        },
        "roofline": {
            "bound": bound,
            "achieved": achieved,
            "peak": peak,
            "unit": unit,
            "frac": achieved / peak,
            "traffic": (measured_traffic(r["tile_config"])
                        if args.workload == HEADLINE else None),
            "achieved_basis": "median process: 2MNK over the mean of per-launch HIP events",
        },
    }
    if "cpu_baseline" in first:
        out["cpu_baseline"] = first["cpu_baseline"]
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
