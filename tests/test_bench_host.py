"""The benchmark's host logic, without a GPU: argument refusals, the JSON line it builds
from its measurements (the contract fields, the median process, the roofline fraction,
the traffic record's guard, the parity gate) and the engine-clock arithmetic."""
import argparse
import io
import json
import os
import subprocess
import sys
from contextlib import redirect_stdout

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from tiled_dense_gemm_major_amd.inputs import WORKLOADS  # noqa: E402


def _bench(*argv):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv],
                          capture_output=True, text=True, timeout=120)


def test_refuses_more_than_one_gpu():
    r = _bench("--gpus", "2")
    assert r.returncode == 2 and "one GPU" in r.stderr and r.stdout == ""


@pytest.mark.parametrize("argv", [("--steps", "0"), ("--warmup", "-1"), ("--procs", "0")])
def test_refuses_bad_counts(argv):
    assert _bench(*argv).returncode == 2


def _recorded_tile_config():
    with open(bench.TRAFFIC_FILE) as f:
        return json.load(f)["tile_config"]


def _result(total_ms, steps, clock, tile_config, parity=None):
    r = {"total_ms": total_ms, "per_launch_ms": [total_ms / steps] * steps,
         "clock_mhz": clock, "clock_spread": [clock - 50, clock - 40, clock + 40, clock + 50, 256],
         "tile_config": tile_config, "device": "test"}
    if parity is not None:
        r["parity"] = parity
        r["cpu_baseline"] = {"value": 0.06, "unit": "TFLOP/s", "cores": 16, "kind": "oracle",
                             "sample": "test"}
    return r


def _report(results, steps=50, workload=bench.HEADLINE):
    args = argparse.Namespace(steps=steps, warmup=10, workload=workload)
    buf = io.StringIO()
    with redirect_stdout(buf):
        bench.report(args, WORKLOADS[workload], results)
    lines = buf.getvalue().strip().splitlines()
    assert len(lines) == 1                      # one JSON line on stdout
    return json.loads(lines[0])


def test_report_contract_and_median_process():
    cfg = _recorded_tile_config()
    ok = {"n_fail": 0, "rows_checked": 8, "elements": 65536, "max_err": 0.0,
          "max_err_over_tol": 0.0}
    # three processes: 36, 35 and 37 ms over 50 steps; the median process is the 36 ms one
    res = [_result(36.0, 50, 1700, cfg, ok), _result(35.0, 50, 1750, cfg),
           _result(37.0, 50, 1650, cfg)]
    out = _report(res)
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline"):
        assert key in out, key
    flops = 2 * 8192 ** 3
    assert out["n_gpus"] == 1 and out["steps"] == 50 and out["warmup"] == 10
    assert out["unit"] == "TFLOP/s" and out["higher_is_better"] is True
    assert out["dtype"] == "bf16" and out["config"]["workload"].startswith("bf16")
    assert out["ms_per_step"] == pytest.approx(36.0 / 50)
    assert out["value"] == pytest.approx(flops / (36.0 / 50 * 1e-3) / 1e12)
    assert out["config"]["engine_clock_mhz"] == 1700
    rl = out["roofline"]
    assert rl["bound"] == "mfma" and rl["unit"] == "TFLOP/s" and rl["peak"] == 2500.0
    assert rl["frac"] == pytest.approx(rl["achieved"] / rl["peak"])
    assert rl["achieved"] == pytest.approx(flops / (36.0 / 50 * 1e-3) / 1e12)
    # the committed traffic record applies to the configuration it was taken on
    assert rl["traffic"] == pytest.approx(bench.measured_traffic(cfg)) and rl["traffic"] > 0
    assert out["cpu_baseline"]["kind"] == "oracle"
    assert out["vs_baseline"] is None


def test_report_traffic_only_for_the_recorded_configuration():
    cfg = dict(_recorded_tile_config(), group_m=_recorded_tile_config()["group_m"] + 1)
    out = _report([_result(36.0, 50, 1700, cfg)])
    assert out["roofline"]["traffic"] is None
    assert bench.measured_traffic(cfg) is None


def test_report_stops_on_a_parity_failure():
    bad = {"n_fail": 3, "rows_checked": 8, "elements": 65536, "max_err": 1.0,
           "max_err_over_tol": 9.0}
    with pytest.raises(SystemExit) as e:
        _report([_result(36.0, 50, 1700, _recorded_tile_config(), bad)])
    assert e.value.code == 1


def test_engine_clock():
    hz = 100e6                                        # a 100 MHz wall clock
    before = [[0, 0]] * 8
    after = [[0, 0]] * 8
    # compute units 0-4 stamped twice: 1000 wall ticks (10 us) and 15, 16, 17, 18, 19
    # thousand engine cycles (1.5-1.9 GHz); unit 5 stamped only before, 6 only after
    for u, cyc in enumerate((15000, 16000, 17000, 18000, 19000)):
        before[u] = [1000 * u, 500]
        after[u] = [1000 * u + cyc, 1500]
    before[5] = [7, 9]
    after[6] = [7, 9]
    med, spread = bench.engine_clock(before, after, hz)
    assert med == pytest.approx(1700.0)
    assert spread == pytest.approx([1500.0, 1500.0, 1900.0, 1900.0, 5])
    assert bench.engine_clock([[0, 0]], [[0, 0]], hz) == (None, None)
