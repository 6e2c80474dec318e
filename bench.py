#!/usr/bin/env python3
"""Benchmark of libtgemm's hot path: one step = one C = A x B^T product of the headline
workload (bf16, M = N = K = 8192, A [M,K] and B [N,K] K-major, inputs uniform[-1,1]
rounded to bf16 from SplitMix64 seed 3, fp32 sums, bf16 output), inputs resident in HBM.

Prints ONE JSON line (stdout).  Progress goes to stderr.

  python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--no-cpu-baseline]

Timing: HIP events recorded on the stream the kernel is launched on, around exactly
`steps` back-to-back launches after `warmup` untimed ones, with device synchronisation
on both sides.  (Parity with the CPU oracle is the test suite's job.)  The CPU baseline
times the oracle on a bounded sample (leading rows of C) on the host cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from tiled_dense_gemm_major_amd import roofline  # noqa: E402
from tiled_dense_gemm_major_amd.profsum import kernel_digest  # noqa: E402
from tiled_dense_gemm_major_amd.inputs import BF16, WORKLOADS  # noqa: E402

HEADLINE = "bf16_8192"
METRIC = "GEMM TFLOP/s at 8192^3 bf16 K-major (1 MI355X) and % of MFMA peak"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gemm_quad_bf16_8192.json")


def log(msg: str):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def measured_traffic():
    """HBM bytes per launch from the committed rocprofv3 counter runs, or None when the
    kernel sources changed since they were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_digest") != kernel_digest():
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(A, B, w, budget_s: float):
    """The oracle (as it is) on the leading rows of C, sized to ~budget_s seconds."""
    import oracle
    cores = oracle.max_threads()
    probe_rows = 64
    t0 = time.perf_counter()
    oracle.gemm_rows(w.dtype, A, B, w.b_layout, 0, probe_rows)
    t_probe = time.perf_counter() - t0
    rows = int(max(probe_rows, min(w.M, probe_rows * budget_s / max(t_probe, 1e-3))))
    log(f"cpu baseline: {probe_rows} rows took {t_probe:.2f}s; timing {rows} rows on "
        f"{cores} threads")
    t0 = time.perf_counter()
    oracle.gemm_rows(w.dtype, A, B, w.b_layout, 0, rows)
    dt = time.perf_counter() - t0
    flops = roofline.gemm_flops(rows, w.N, w.K)
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": cores,
        "kind": "oracle",
        "sample": (f"rows 0..{rows - 1} of C ({rows}x{w.N} outputs, full K={w.K}) of the "
                   f"{w.describe()} product; {dt:.1f} s including decode and rounding"),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=HEADLINE, choices=list(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget-s", type=float, default=15.0)
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the product "
              f"is a single-device kernel library and no multi-GPU path is built.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from tiled_dense_gemm_major_amd import tgemm

    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        sys.exit(1)
    tgemm.load()

    w = WORKLOADS[args.workload]
    log(f"workload {w.describe()}")
    A_bits, B_bits = w.generate()
    tdt = torch.bfloat16 if w.dtype == BF16 else torch.float16
    A = torch.from_numpy(A_bits.view(np.int16)).cuda().view(tdt)
    B = torch.from_numpy(B_bits.view(np.int16)).cuda().view(tdt)
    C = torch.empty((w.M, w.N), dtype=tdt, device="cuda")
    cfg = tgemm.query_config(w.dtype, w.M, w.N, w.K, w.b_layout)
    stream = torch.cuda.current_stream()

    def step():
        tgemm.gemm_ex(w.dtype, w.M, w.N, w.K, A, B, C, w.b_layout, None, stream)

    step()
    torch.cuda.synchronize()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    per = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record(stream)
    for ev0, ev1 in per:
        ev0.record(stream)
        step()
        ev1.record(stream)
    stop.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = start.elapsed_time(stop)
    per_ms = sorted(a.elapsed_time(b) for a, b in per)
    ms_per_step = total_ms / args.steps
    median_ms = per_ms[len(per_ms) // 2]

    flops = roofline.gemm_flops(w.M, w.N, w.K)
    dname = "bf16" if w.dtype == BF16 else "f16"
    tflops = flops / (ms_per_step * 1e-3) / 1e12
    peak_tflops = roofline.PEAK_FLOPS[dname] / 1e12
    bound = roofline.bound(w.M, w.N, w.K, dname)
    # the kernel's own rate: algorithmic work of one launch over the average launch
    # duration (HIP events around each launch, on the launch stream)
    launch_ms = sum(per_ms) / len(per_ms)
    if bound == "mfma":
        achieved = flops / (launch_ms * 1e-3) / 1e12
        peak, unit = peak_tflops, "TFLOP/s"
    else:
        achieved = roofline.compulsory_bytes(w.M, w.N, w.K) / (launch_ms * 1e-3) / 1e9
        peak, unit = roofline.HBM_BYTES_PER_S / 1e9, "GB/s"
    log(f"{args.steps} steps: {total_ms:.3f} ms total, {ms_per_step * 1e3:.1f} us/step "
        f"(median {median_ms * 1e3:.1f} us), {tflops:.1f} TFLOP/s, wall {wall:.3f} s")

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
            "workload": w.describe() + " C=A*B^T" if w.b_layout == 0 else w.describe(),
            "M": w.M, "N": w.N, "K": w.K,
            "b_layout": "NK" if w.b_layout == 0 else "KN",
            "tile_config": cfg.as_dict(),
            "median_ms_per_step": median_ms,
            "avg_ms_per_launch": launch_ms,
            "frac_of_mfma_peak": tflops / peak_tflops,
        },
        "roofline": {
            "bound": bound,
            "achieved": achieved,
            "peak": peak,
            "unit": unit,
            "frac": achieved / peak,
            "traffic": measured_traffic(),
        },
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(A_bits, B_bits, w, args.cpu_budget_s)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
