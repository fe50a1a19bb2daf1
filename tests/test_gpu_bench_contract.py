"""Every benchmark workload prints one well-formed JSON line on the GPU: the
fields of the benchmark contract, a roofline object whose fraction is its
achieved rate over its peak, and (default line only) the CPU baseline.  Short
runs: two timed steps, no clock settling."""

import json
import math
import os
import subprocess
import sys

import pytest

from tests.gpu_util import say

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
WORKLOADS = ["dense", "quant", "moe", "moe_ep", "wgrad", "dgrad", "pow2", "fused", "tiny", "pertensor"]


def _bench(args):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                       cwd=ROOT, timeout=240)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, f"expected one line, got {len(lines)}"
    return json.loads(lines[0])


def _check_contract(d, steps, warmup):
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
              "scaling", "vs_baseline", "dtype", "data", "config", "roofline"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == steps and d["warmup"] == warmup
    # rates are higher-is-better; the small case reports a latency
    assert d["higher_is_better"] is (d["unit"] not in ("us", "ms"))
    assert d["scaling"] == "weak" and d["data"] == "synthetic"
    assert math.isfinite(d["value"]) and d["value"] > 0 and d["ms_per_step"] > 0
    assert isinstance(d["config"].get("workload"), str) and "model" not in d["config"]
    r = d["roofline"]
    assert r["bound"] in ("hbm", "mfma") and r["unit"] == ("GB/s" if r["bound"] == "hbm" else "TFLOP/s")
    # HBM 8 TB/s; dense FP8 5.0 PFLOP/s, or fp16 2.5 for the exact (fp16-widened) GEMMs
    assert r["peak"] in ((8000.0,) if r["bound"] == "hbm" else (5000.0, 2500.0))
    assert r["achieved"] > 0 and abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-9
    assert "traffic" in r


@pytest.mark.timeout(1200)
@pytest.mark.parametrize("workload", WORKLOADS)
def test_workload_line(workload):
    say(f"bench.py --workload {workload} --steps 2 --warmup 1 --settle 0 --no-cpu-baseline")
    d = _bench(["--workload", workload, "--steps", "2", "--warmup", "1", "--settle", "0", "--no-cpu-baseline"])
    _check_contract(d, 2, 1)


@pytest.mark.timeout(600)
def test_default_line_carries_the_cpu_baseline():
    say("bench.py --steps 2 --warmup 1 --settle 0 (default line, with the CPU baseline)")
    d = _bench(["--steps", "2", "--warmup", "1", "--settle", "0"])
    _check_contract(d, 2, 1)
    c = d["cpu_baseline"]
    assert c["kind"] == "oracle" and c["value"] > 0 and c["cores"] >= 1 and c["sample"]
    assert d["dtype"] == "e4m3" and d["roofline"]["bound"] == "mfma"
