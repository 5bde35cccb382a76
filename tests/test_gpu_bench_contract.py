"""The benchmark's output contract: one JSON line with the metric, value, timing, roofline and CPU
baseline fields, on a small grid (a short run of bench.py in a child process on the GPU)."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("workload", ["s4", "s4s", "j_small", "b_mid"])
def test_bench_prints_one_contract_line(workload):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", workload, "--steps", "2",
                        "--warmup", "1"], capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, lines
    res = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert key in res, key
    assert res["n_gpus"] == 1 and res["steps"] == 2 and res["warmup"] == 1 and res["value"] > 0
    assert "workload" in res["config"]
    roof = res["roofline"]
    for key in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert key in roof, key
    assert roof["bound"] in ("mfma", "hbm") and 0 < roof["frac"] < 1
    cpu = res["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["cores"] >= 1 and cpu["value"] > 0 and cpu["sample"]
    # per-step timings: mean, median and min of the event-timed calls
    timings = res["call_ms"] if not workload.startswith("b_") else next(iter(res["call_ms"].values()))
    assert 0 < timings["min"] <= timings["median"] and timings["min"] <= timings["mean"]
    # the graphics clock sampled during the timed steps (sysfs or amdsmi)
    assert "sclk" in res
    if res["sclk"] is not None:
        assert 0 < res["sclk"]["min_mhz"] <= res["sclk"]["mean_mhz"] <= res["sclk"]["max_mhz"] < 5000
        assert res["sclk"]["samples"] >= 1 and res["sclk"]["source"]
    if not workload.startswith("b_"):
        par = res["parity"]
        assert par["max_abs"] <= 2e-2 and par["rel_l2"] <= 1e-2, par
    if workload == "s4s":
        chk = res["parity"]["router_mask_vs_oracle"]
        assert chk["head"] == 0 and chk["rows"] == 38 and chk["rows_mismatched"] == 0
        assert res["route_call_ms"]["min"] > 0


def test_bench_refuses_several_gpus():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode != 0 and "one GPU" in r.stderr
