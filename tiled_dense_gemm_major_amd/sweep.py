"""Tile-configuration sweep: time every configuration compiled into libtgemm on a set of
workloads and report the fastest per workload -- the search whose frozen result is the
library's per-shape table (autotuning over block sizes and pipeline depth, as in the Tilus
tutorial's autotune space and the TileLang page's advice to freeze the results per
machine into a configuration table).

  python -m tiled_dense_gemm_major_amd.sweep [--workloads a,b] [--repeat 20] [--warmup 5]
  python -m tiled_dense_gemm_major_amd.sweep --copy-bytes 536870912 --repeat 5

The second form runs only a plain device-to-device copy of a known size: the reference
against which hardware byte counters (FETCH_SIZE, WRITE_SIZE) are scaled.

Prints one JSON line per (workload, configuration): median/p10/p90 microseconds from HIP
events on the launch stream, TFLOP/s, fraction of the MFMA peak and of the HBM roofline.
"""
from __future__ import annotations

import argparse
import json
import sys

from . import roofline
from .inputs import BF16, WORKLOADS


def time_config(tgemm, torch, w, A, B, C, cfg, warmup, repeat, stream):
    def go():
        tgemm.gemm_ex(w.dtype, w.M, w.N, w.K, A, B, C, w.b_layout, cfg, stream)
    for _ in range(warmup):
        go()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(repeat)]
    for a, b in evs:
        a.record(stream)
        go()
        b.record(stream)
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) * 1e3 for a, b in evs)
    return t[len(t) // 2], t[len(t) // 10], t[(9 * len(t)) // 10]


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--workloads", default=",".join(WORKLOADS))
    ap.add_argument("--repeat", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--copy-bytes", type=int, default=0)
    ap.add_argument("--torch-ref", action="store_true",
                    help="also time torch.matmul (the vendor library) as context")
    ap.add_argument("--kernels", default="",
                    help="comma-separated kernel ids to time (default: every compiled one)")
    args = ap.parse_args(argv)

    import numpy as np
    import torch

    if args.copy_bytes:
        src = torch.ones(args.copy_bytes // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(args.repeat):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": args.copy_bytes, "launches": args.repeat}))
        return

    from . import tgemm
    tgemm.load()
    stream = torch.cuda.current_stream()
    best = {}
    for name in args.workloads.split(","):
        w = WORKLOADS[name]
        A_bits, B_bits = w.generate()
        tdt = torch.bfloat16 if w.dtype == BF16 else torch.float16
        A = torch.from_numpy(A_bits.view(np.int16)).cuda().view(tdt)
        B = torch.from_numpy(B_bits.view(np.int16)).cuda().view(tdt)
        C = torch.empty((w.M, w.N), dtype=tdt, device="cuda")
        dname = "bf16" if w.dtype == BF16 else "f16"
        flops = roofline.gemm_flops(w.M, w.N, w.K)
        nbytes = roofline.compulsory_bytes(w.M, w.N, w.K)
        table = tgemm.query_config(w.dtype, w.M, w.N, w.K, w.b_layout).as_dict()
        kernels = {int(x) for x in args.kernels.split(",") if x}
        for cfg in tgemm.list_configs(w.dtype, w.b_layout):
            if kernels and cfg.kernel not in kernels:
                continue
            med, p10, p90 = time_config(tgemm, torch, w, A, B, C, cfg, args.warmup,
                                        args.repeat, stream)
            rec = {
                "workload": name, "config": cfg.as_dict(), "table_choice":
                cfg.as_dict() == table, "median_us": med, "p10_us": p10, "p90_us": p90,
                "tflops": flops / med / 1e6,
                "frac_mfma_peak": flops / med / 1e6 / (roofline.PEAK_FLOPS[dname] / 1e12),
                "gbps": nbytes / med / 1e3,
                "frac_hbm": nbytes / med / 1e3 / (roofline.HBM_BYTES_PER_S / 1e9),
            }
            print(json.dumps(rec), flush=True)
            if name not in best or med < best[name]["median_us"]:
                best[name] = rec
        if args.torch_ref:
            Bt = B.t() if w.b_layout == 0 else B     # the [K, N] operand either way
            def ref():
                torch.matmul(A, Bt, out=C)
            for _ in range(args.warmup):
                ref()
            torch.cuda.synchronize()
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(args.repeat)]
            for a, b in evs:
                a.record(stream)
                ref()
                b.record(stream)
            torch.cuda.synchronize()
            t = sorted(a.elapsed_time(b) * 1e3 for a, b in evs)
            med = t[len(t) // 2]
            print(json.dumps({"workload": name, "config": "torch.matmul (vendor library)",
                              "median_us": med, "tflops": flops / med / 1e6}), flush=True)
        del A, B, C
        torch.cuda.empty_cache()
    for name, rec in best.items():
        print(f"best {name}: {rec['config']} {rec['median_us']:.1f} us "
              f"{rec['tflops']:.1f} TFLOP/s", file=sys.stderr)


if __name__ == "__main__":
    main()
