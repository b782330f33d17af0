"""bench.py's output line on the GPU: every field of the JSON contract, the
roofline computed from the per-launch event times, and the CPU baseline leg,
on two small workloads (a few timed steps each)."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args):
    print("bench.py", *args, flush=True)
    r = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.startswith("{")]
    assert len(lines) == 1, r.stdout[-2000:]
    return json.loads(lines[0])


def _common(d, workload, steps, warmup):
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == steps and d["warmup"] == warmup
    assert d["unit"] == "params/s" and d["higher_is_better"] is True and d["scaling"] == "weak"
    assert d["dtype"] == "f32" and d["data"] == "synthetic" and d["vs_baseline"] is None
    assert d["config"]["workload"] == workload
    n = d["config"]["n_elems"]
    assert d["value"] > 0 and abs(d["value"] - n / (d["ms_per_step"] / 1e3)) <= 1e-6 * d["value"]


def test_bench_line_vit_b_set_with_roofline():
    d = _bench("--workload", "vit-b-set-demo-k1", "--steps", "4", "--warmup", "1", "--no-cpu-baseline")
    _common(d, "vit-b-set-demo-k1", 4, 1)
    r = d["roofline"]
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    k = d["kernels"][r["kernel"]]
    assert k["calls"] == 4
    # achieved = algorithmic bytes per launch over the average launch time
    assert abs(r["achieved"] - k["bytes"] / (k["avg_ms"] / 1e3) / 1e9) <= 1e-6 * r["achieved"]
    assert abs(r["frac"] - r["achieved"] / r["peak"]) <= 1e-12
    assert 0.0 < r["frac"] < 1.0
    assert d["cpu_baseline"] is None


def test_bench_line_launch_bound_tensor_with_cpu_baseline():
    d = _bench("--workload", "tensor-4096-demo-k4", "--steps", "3", "--warmup", "1", "--cpu-seconds", "1")
    _common(d, "tensor-4096-demo-k4", 3, 1)
    assert d["roofline"] is None and "launch_bound" in d
    c = d["cpu_baseline"]
    assert c["kind"] == "oracle" and c["unit"] == "params/s" and c["value"] > 0 and c["cores"] >= 1
    assert isinstance(c["sample"], str) and c["sample"]
    assert c["single_core"]["cores"] == 1 and c["single_core"]["value"] > 0
