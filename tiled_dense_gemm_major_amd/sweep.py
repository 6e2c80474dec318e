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

  --cold N     rotate over N separately allocated copies of A and B, one per launch, so
               that (with N copies larger than the 256 MB last-level cache) every launch
               reads its operands from HBM;
  --rounds R   time the configurations (and the vendor library) in R interleaved rounds
               of --repeat launches each, so that slow drifts of the clock (the chip is
               power-limited) fall on every configuration alike.

  python -m tiled_dense_gemm_major_amd.sweep --emit-table tiled_dense_gemm_major_amd/csrc/tile_table.inc

refreshes the library's frozen per-device table: every fast configuration is timed on a
grid of shapes (A [M,K], B [N,K] and [K,N]; bf16, whose kernels are fp16's too), and the
fastest per grid point is written as a C++ table that `choose` consults (the nearest grid
point in log2 of M, N and K) before its fallback rules.  Rebuild the library afterwards.
With --layouts kn (or nk) only that half is re-timed and the rest kept from the file;
--table-ms 16,64 likewise limits the re-timing to those rows of M.

  python -m tiled_dense_gemm_major_amd.sweep --attention [--repeat 20]

times the attention forward pass (attn_fwd_f16) on its workloads instead: median/p10/p90
microseconds, TFLOP/s over the (query, key) pairs the mask keeps, and the fractions of the
fp16 MFMA peak and of the HBM roofline (Q, K, V read once, O written once).
"""
from __future__ import annotations

import argparse
import json
import sys

from . import roofline
from .inputs import B_KN, B_NK, BF16, F16, WORKLOADS, Workload


def time_launches(torch, fn, n, stream):
    """Durations (us) of n launches of fn, each bracketed by HIP events on the stream."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n)]
    for i, (a, b) in enumerate(evs):
        a.record(stream)
        fn(i)
        b.record(stream)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) * 1e3 for a, b in evs]


def summary(t):
    t = sorted(t)
    return t[len(t) // 2], t[len(t) // 10], t[(9 * len(t)) // 10]


# The table's grid: powers of two and, for M and N, the points half-way between them in
# log2 (x 1.5), where tiles of 192 rows or 128 columns can fill the chip better than
# 256-wide ones; plus the small M of decode-like products.
TABLE_M = (16, 64, 128, 256, 512, 768, 1024, 1536, 2048, 3072, 4096, 6144, 8192)
TABLE_N = (512, 768, 1024, 1536, 2048, 3072, 4096, 6144, 8192)
TABLE_K = (512, 1024, 2048, 4096, 8192)


def read_table(path):
    """Entries of an existing table file: (layout, mi, ni, ki) -> (config dict, us)."""
    import re
    names = ["kernel", "block_m", "block_n", "block_k", "waves_m", "waves_n", "stages",
             "group_m", "split_k", "mfma"]
    out = {}
    with open(path) as f:
        for m in re.finditer(r"\{(\d+), (\d+), (\d+), (\d+), \{([-\d, ]+)\}\},\s*//\s*([\d.]+)",
                             f.read()):
            key = tuple(int(m.group(i)) for i in range(1, 5))
            out[key] = (dict(zip(names, (int(v) for v in m.group(5).split(",")))),
                        float(m.group(6)))
    return out


def emit_table(tgemm, torch, np, args, stream, path):
    """Time every fast configuration on the grid and write the fastest per point.  With
    --layouts (and --table-ms), only those B storages (and M rows) are timed; the other
    rows are kept from the file."""
    import datetime
    from .inputs import B_KN, B_NK
    layouts = [B_NK, B_KN] if not args.layouts else \
        [B_KN if x == "kn" else B_NK for x in args.layouts.split(",")]
    ms = [int(x) for x in args.table_ms.split(",") if x]
    if any(m not in TABLE_M for m in ms):
        raise SystemExit(f"--table-ms: rows of the grid are {TABLE_M}")
    partial = bool(args.layouts or ms)
    kept = read_table(path) if partial else {}
    rows = []
    for layout in (B_NK, B_KN):
        cfgs = [c for c in tgemm.list_configs(BF16, layout)
                if c.kernel not in tgemm.ANY_ALIGNMENT_KERNELS
                and c.kernel not in tgemm.WORKSPACE_KERNELS]
        for mi, M in enumerate(TABLE_M):
            if layout not in layouts or (ms and M not in ms):
                for ni in range(len(TABLE_N)):
                    for ki in range(len(TABLE_K)):
                        d, us = kept[(layout, mi, ni, ki)]
                        rows.append((layout, mi, ni, ki, tgemm.Config.from_dict(d), us))
                continue
            for ni, N in enumerate(TABLE_N):
                for ki, K in enumerate(TABLE_K):
                    # uniform[-1,1) operands drawn on the device (timing only)
                    A = torch.empty((M, K), dtype=torch.bfloat16,
                                    device="cuda").uniform_(-1.0, 1.0)
                    shape_b = (N, K) if layout == B_NK else (K, N)
                    B = torch.empty(shape_b, dtype=torch.bfloat16,
                                    device="cuda").uniform_(-1.0, 1.0)
                    C = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
                    runs = []
                    for c in cfgs:
                        def go(i, c=c):
                            tgemm.gemm_ex(BF16, M, N, K, A, B, C, layout, c, stream)
                        runs.append((c, go))
                    times = [[] for _ in runs]
                    for _, fn in runs:
                        for i in range(args.warmup):
                            fn(i)
                    torch.cuda.synchronize()
                    for _ in range(max(1, args.rounds)):
                        for r, (_, fn) in enumerate(runs):
                            times[r] += time_launches(torch, fn, args.repeat, stream)
                    meds = [summary(t)[0] for t in times]
                    best = int(np.argmin(meds))
                    c = runs[best][0]
                    rows.append((layout, mi, ni, ki, c, meds[best]))
                    print(json.dumps({"layout": layout, "M": M, "N": N, "K": K,
                                      "best": c.as_dict(), "median_us": meds[best]}),
                          flush=True)
                    del A, B, C
    dev = torch.cuda.get_device_properties(0)
    lines = [
        "// Frozen per-device configuration table (generated; do not edit by hand).",
        f"// Device: {dev.name} ({getattr(dev, 'gcnArchName', 'gfx950')}), "
        f"{datetime.date.today().isoformat()}; bf16, warmup {args.warmup}, "
        f"{max(1, args.rounds)} x {args.repeat} launches per configuration, medians"
        + (f"; re-timed: {args.layouts or 'nk,kn'} rows"
           + (f" at M {args.table_ms}" if ms else "")
           + ", the others kept from the previous table." if partial else "."),
        "// Regenerate: python -m tiled_dense_gemm_major_amd.sweep --emit-table <this file>",
        "static const int64_t kTableM[] = {" + ", ".join(map(str, TABLE_M)) + "};",
        "static const int64_t kTableN[] = {" + ", ".join(map(str, TABLE_N)) + "};",
        "static const int64_t kTableK[] = {" + ", ".join(map(str, TABLE_K)) + "};",
        "// {b_layout, m index, n index, k index, {config}}  (median us when measured)",
        "static const TableEntry kTable[] = {",
    ]
    for layout, mi, ni, ki, c, us in rows:
        d = c.as_dict()
        lines.append(
            f"    {{{layout}, {mi}, {ni}, {ki}, {{{d['kernel']}, {d['block_m']}, {d['block_n']}, "
            f"{d['block_k']}, {d['waves_m']}, {d['waves_n']}, {d['stages']}, {d['group_m']}, "
            f"{d['split_k']}, {d['mfma']}}}}},  // {us:.1f}")
    lines.append("};")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(f"wrote {path}: {len(rows)} entries", file=sys.stderr)


def time_attention(tgemm, torch, np, args, stream):
    from .inputs import ATTN_WORKLOADS
    for name, w in ATTN_WORKLOADS.items():
        Q, K, V = (torch.from_numpy(x.view(np.int16)).cuda().view(torch.float16)
                   for x in w.generate())
        O = torch.empty_like(Q)
        B, S, H, D = w.shape

        def go(i):
            tgemm.attn_fwd_f16(B, S, H, D, Q, K, V, O, w.causal, stream)
        for i in range(args.warmup):
            go(i)
        torch.cuda.synchronize()
        t = []
        for _ in range(max(1, args.rounds)):
            t += time_launches(torch, go, args.repeat, stream)
        med, p10, p90 = summary(t)
        flops = roofline.attention_flops(B, S, H, D, w.causal)
        nbytes = roofline.attention_bytes(B, S, H, D)
        print(json.dumps({
            "workload": name, "kernel": "attn_fwd_f16", "median_us": med, "p10_us": p10,
            "p90_us": p90, "tflops": flops / med / 1e6,
            "frac_mfma_peak": flops / med / 1e6 / (roofline.PEAK_FLOPS["f16"] / 1e12),
            "gbps": nbytes / med / 1e3,
            "frac_hbm": nbytes / med / 1e3 / (roofline.HBM_BYTES_PER_S / 1e9),
            "launches": len(t)}), flush=True)
        del Q, K, V, O
        torch.cuda.empty_cache()


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--workloads", default=",".join(WORKLOADS))
    ap.add_argument("--repeat", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--copy-bytes", type=int, default=0)
    ap.add_argument("--cold", type=int, default=0,
                    help="rotate over this many copies of A and B (HBM-resident operands)")
    ap.add_argument("--emit-table", default="",
                    help="time the grid and write the frozen configuration table here")
    ap.add_argument("--table-ms", default="",
                    help="with --emit-table: re-time only these M rows of the grid "
                         "(e.g. 16,64), keeping the others from the file")
    ap.add_argument("--layouts", default="",
                    help="with --emit-table: re-time only these B storages (nk, kn), "
                         "keeping the file's other rows")
    ap.add_argument("--attention", action="store_true",
                    help="time the attention forward pass on its workloads instead")
    ap.add_argument("--rounds", type=int, default=1,
                    help="interleaved timing rounds of --repeat launches per configuration")
    ap.add_argument("--torch-ref", action="store_true",
                    help="also time torch.matmul (the vendor library) as context")
    ap.add_argument("--table-only", action="store_true",
                    help="time only the table's choices (without and with a workspace)")
    ap.add_argument("--splits", default="",
                    help="comma-separated split counts to time for the split-K kernels "
                         "(default: the table's count with a workspace and its neighbours)")
    ap.add_argument("--kernels", default="",
                    help="comma-separated kernel ids to time (default: every compiled one)")
    ap.add_argument("--shapes", default="",
                    help="extra products to time, comma-separated DTYPE:MxNxK:LAYOUT[:km] "
                         "(e.g. bf16:8192x8192x8192:kn; :km stores A as [K,M]), inputs "
                         "U[-1,1] from seed 0")
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
    if args.attention:
        time_attention(tgemm, torch, np, args, stream)
        return
    if args.emit_table:
        emit_table(tgemm, torch, np, args, stream, args.emit_table)
        return
    best = {}
    todo = [(name, WORKLOADS[name], 0) for name in args.workloads.split(",") if name]
    for spec in [x for x in args.shapes.split(",") if x]:
        parts = spec.split(":")
        dt, mnk, lay = parts[:3]
        a_km = len(parts) > 3 and parts[3] == "km"      # A stored [K,M]
        M, N, K = (int(v) for v in mnk.split("x"))
        todo.append((spec, Workload(spec, BF16 if dt == "bf16" else F16, M, N, K,
                                    B_KN if lay == "kn" else B_NK, "uniform", 0),
                     1 if a_km else 0))
    for name, w, a_layout in todo:
        A_bits, B_bits = w.generate()
        tdt = torch.bfloat16 if w.dtype == BF16 else torch.float16
        copies = max(1, args.cold)
        if a_layout:                                    # A stored [K,M]
            A_bits = np.ascontiguousarray(A_bits.T)
        As = [torch.from_numpy(A_bits.view(np.int16)).cuda().view(tdt) for _ in range(copies)]
        Bs = [torch.from_numpy(B_bits.view(np.int16)).cuda().view(tdt) for _ in range(copies)]
        C = torch.empty((w.M, w.N), dtype=tdt, device="cuda")
        dname = "bf16" if w.dtype == BF16 else "f16"
        flops = roofline.gemm_flops(w.M, w.N, w.K)
        nbytes = roofline.compulsory_bytes(w.M, w.N, w.K)
        # packed operands meet the fast kernels' rules when every row length is a
        # multiple of 8 elements (the allocations themselves are aligned)
        aligned = w.K % 8 == 0 and w.N % 8 == 0 and (not a_layout or w.M % 8 == 0)
        if not aligned and w.K % 8 == 0 and w.b_layout == B_NK and not a_layout:
            aligned = tgemm.ALIGN_OPERANDS              # A and B meet them, N does not
        operands_only = aligned is not True and aligned == tgemm.ALIGN_OPERANDS
        allowed = tgemm.ANY_ALIGNMENT_KERNELS + ((tgemm.KERNEL_SKINNY,) if operands_only else ())
        table = tgemm.query_config(w.dtype, w.M, w.N, w.K, w.b_layout, aligned,
                                   a_layout).as_dict()
        table_ws = tgemm.query_config_ws(w.dtype, w.M, w.N, w.K, w.b_layout,
                                         aligned)[0].as_dict()
        kernels = {int(x) for x in args.kernels.split(",") if x}

        runners = []
        ws_cfg, _ = tgemm.query_config_ws(w.dtype, w.M, w.N, w.K, w.b_layout, aligned)
        lda = w.M if a_layout else w.K
        ldb = w.N if w.b_layout == B_KN else w.K
        for cfg in tgemm.list_configs(w.dtype, w.b_layout, a_layout):
            if kernels and cfg.kernel not in kernels:
                continue
            if aligned is not True and cfg.kernel not in allowed:
                continue                                # the fast kernels refuse these
            if a_layout:                                # the general entry point
                def go(i, c=cfg):
                    tgemm.gemm_strided(w.dtype, w.M, w.N, w.K, As[i % copies], lda,
                                       a_layout, Bs[i % copies], ldb, w.b_layout, C, w.N,
                                       c, stream)
                if not args.table_only or cfg.as_dict() == table:
                    runners.append((cfg, go))
                continue
            if cfg.kernel in tgemm.SPLIT_KERNELS:
                # split counts: the table's (with a workspace) and its neighbours
                base = ws_cfg.split_k if ws_cfg.kernel == cfg.kernel else 8
                counts = ([int(x) for x in args.splits.split(",") if x] if args.splits
                          else [max(2, base // 2), base, min(64, base * 2)])
                variants = []
                for sk in sorted(set(counts)):
                    c = tgemm.Config.from_dict({**cfg.as_dict(), "split_k": sk})
                    variants.append(c)
            else:
                variants = [cfg]
            for c in variants:
                if args.table_only and c.as_dict() not in (table, table_ws):
                    continue
                ws_bytes = tgemm.workspace_size(w.M, w.N, c)
                ws = torch.empty((max(ws_bytes, 16),), dtype=torch.uint8, device="cuda")
                def go(i, c=c, ws=ws, ws_bytes=ws_bytes):
                    tgemm.gemm_ex_ws(w.dtype, w.M, w.N, w.K, As[i % copies],
                                     Bs[i % copies], C, ws, ws_bytes, w.b_layout, c, stream)
                runners.append((c, go))
        if args.torch_ref:
            # the [K, N] operand either way
            Bts = [B.t() if w.b_layout == 0 else B for B in Bs]
            def ref(i):
                torch.matmul(As[i % copies], Bts[i % copies], out=C)
            runners.append((None, ref))

        times = [[] for _ in runners]
        for _, fn in runners:
            for i in range(args.warmup):
                fn(i)
        torch.cuda.synchronize()
        for _ in range(max(1, args.rounds)):
            for r, (_, fn) in enumerate(runners):
                times[r] += time_launches(torch, fn, args.repeat, stream)
        for (cfg, _), t in zip(runners, times):
            med, p10, p90 = summary(t)
            rec = {
                "workload": name,
                "config": cfg.as_dict() if cfg is not None else "torch.matmul (vendor library)",
                "table_choice": cfg is not None and cfg.as_dict() == table,
                "table_choice_ws": cfg is not None and cfg.as_dict() == table_ws,
                "median_us": med, "p10_us": p10, "p90_us": p90,
                "tflops": flops / med / 1e6,
                "frac_mfma_peak": flops / med / 1e6 / (roofline.PEAK_FLOPS[dname] / 1e12),
                "gbps": nbytes / med / 1e3,
                "frac_hbm": nbytes / med / 1e3 / (roofline.HBM_BYTES_PER_S / 1e9),
                "cold_copies": args.cold, "launches": len(t),
            }
            print(json.dumps(rec), flush=True)
            if cfg is not None and (name not in best or med < best[name]["median_us"]):
                best[name] = rec
        del As, Bs, C
        torch.cuda.empty_cache()
    for name, rec in best.items():
        print(f"best {name}: {rec['config']} {rec['median_us']:.1f} us "
              f"{rec['tflops']:.1f} TFLOP/s", file=sys.stderr)


if __name__ == "__main__":
    main()
