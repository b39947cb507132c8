"""The benchmark's output contract on the GPU: one JSON line with the metric,
the roofline of the dominant kernel and the CPU-oracle baseline, here on the
tiny workload (one layer, two heads of 64, fp32; the small configuration the
oracle finishes at once), run as its own process as a user would."""
import json
import os
import subprocess
import sys

import pytest

import bench

pytestmark = pytest.mark.gpu


def test_bench_json_line_on_the_tiny_workload():
    root = os.path.dirname(os.path.abspath(bench.__file__))
    p = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--workload", "tiny",
                        "--steps", "3", "--warmup", "1", "--cpu-seconds", "1"],
                       capture_output=True, text=True, timeout=240, cwd=root)
    assert p.returncode == 0, p.stderr[-2000:]
    lines = [l for l in p.stdout.splitlines() if l.strip()]
    assert len(lines) == 1
    rec = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
              "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config"):
        assert k in rec, k
    assert rec["n_gpus"] == 1 and rec["steps"] == 3 and rec["warmup"] == 1
    assert rec["unit"] == "GB/s" and rec["value"] > 0 and rec["ms_per_step"] > 0
    assert rec["config"]["workload"] == "tiny" and rec["dtype"] == "f32"
    r = rec["roofline"]
    for k in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert k in r, k
    assert r["bound"] == "hbm" and r["peak"] == 8000.0
    assert abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-3
    c = rec["cpu_baseline"]
    for k in ("value", "unit", "cores", "kind", "sample"):
        assert k in c, k
    assert c["kind"] == "oracle" and c["value"] > 0 and c["cores"] >= 1
    assert rec["order_sensitive_tokens"] == 0
