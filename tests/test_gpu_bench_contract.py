"""bench.py's output line on a GPU: one JSON object with the keys its
callers read, the roofline and CPU-baseline objects, and figures that agree
with each other.  Runs the small cache-resident workload (N=8 ranks of 2^20
float32) as a child process, with the secondary measurements off and a short
oracle timing, so it takes seconds."""

import json
import os
import subprocess
import sys

import pytest
import torch

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_prints_one_contract_line():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    run = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "5", "--warmup", "2",
                          "--workload", "uniform_8x1048576_fp32", "--no-secondary", "--cpu-seconds", "0.5"],
                         capture_output=True, text=True, timeout=240, cwd=ROOT)
    assert run.returncode == 0, run.stderr[-3000:]
    lines = [ln for ln in run.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, run.stdout
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 5 and d["warmup"] == 2
    assert d["unit"] == "GB/s" and d["higher_is_better"] is True and d["dtype"] == "f32"
    assert d["config"]["workload"] == "uniform_8x1048576_fp32"
    assert "N=8, M=1048576" in d["metric"]
    # value = the step's algorithmic bytes over the measured time per step
    n, m = 8, 1 << 20
    assert d["config"]["bytes_per_step"] == 2 * (n + 1) * m * 4
    assert d["value"] == pytest.approx(d["config"]["bytes_per_step"] / (d["ms_per_step"] / 1e3) / 1e9, rel=1e-9)
    assert 0 < d["value"] < 1e5
    roof = d["roofline"]
    assert roof["bound"] == "hbm" and roof["unit"] == "GB/s" and roof["peak"] == 8000.0
    assert roof["frac"] == pytest.approx(roof["achieved"] / roof["peak"], rel=1e-9)
    assert roof["kernel"] in ("rs_direct_kernel", "ag_direct_kernel")
    assert roof["achieved"] == pytest.approx(
        roof["algorithmic_bytes_per_launch"] / (roof["avg_launch_ms"] / 1e3) / 1e9, rel=1e-9)
    cpu = d["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["unit"] == "GB/s" and cpu["cores"] == 1 and cpu["value"] > 0
    assert cpu["seconds"] >= 0.5 and cpu["passes"] >= 1
