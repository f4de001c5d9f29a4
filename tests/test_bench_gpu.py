"""bench.py's output contract, on the small single-segment workload: one JSON line with the
metric, value, roofline (bound, achieved, peak, unit, frac, traffic) and the CPU baseline
(value, unit, cores, kind, sample), parity of the GPU step with the oracle on the sample."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("codec", ["topk", "randk"])
def test_bench_json_line(codec):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload",
                        "c1_single_1m", "--codec", codec, "--steps", "3", "--warmup", "1"],
                       capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["higher_is_better"] is True
    assert d["config"]["workload"].startswith("c1_single_1m")
    rf = d["roofline"]
    for key in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert key in rf, key
    assert rf["bound"] == "hbm" and rf["unit"] == "GB/s" and rf["peak"] == 8000.0
    assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
    cb = d["cpu_baseline"]
    for key in ("value", "unit", "cores", "kind", "sample"):
        assert key in cb, key
    assert cb["kind"] == "oracle" and cb["cores"] >= 1
    assert cb["parity_with_gpu_on_sample"] is True
    # the median of the timed steps and the record of the synthetic gradient's bytes
    assert d["median_ms_per_step"] > 0
    assert len(d["gradient_sha256_16"]) == 16
