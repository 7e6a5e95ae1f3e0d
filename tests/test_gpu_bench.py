"""The benchmark's JSON line on the GPU: a short run of the default workload (16-token
block, sampled) with the fp64 oracle baseline, checked for the fields the line carries."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_line():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "3", "--warmup", "2",
                        "--no-extra"], capture_output=True, text=True, timeout=280)
    assert r.returncode == 0, r.stderr[-2000:]
    d = json.loads(r.stdout.strip().splitlines()[-1])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
              "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline", "accepted_tokens_per_sec"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 2
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["unit"] == "positions/s"
    assert "block16" in d["config"]["workload"]
    roof = d["roofline"]
    assert roof["bound"] == "hbm" and roof["unit"] == "GB/s" and roof["peak"] == 8000.0
    assert 0 < roof["frac"] < 1 and roof["frac"] == pytest.approx(roof["achieved"] / roof["peak"])
    cpu = d["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["value"] > 0 and cpu["cores"] >= 1 and cpu["sample"]
    assert cpu["os_cpu_count"] >= 1
    # tau over the rotated input sets, with its interval and the oracle's closed form beside it
    assert d["input_sets"] == 16 and len(d["tau_sets"]) == 16
    lo, hi = d["tau_ci95"]
    assert lo <= d["tau"] <= hi
    assert d["tau_closed_form"]["tau"] >= 1.0
    peaks = d["measured_peaks"]
    assert 1000 < peaks["hbm_read_GBps"] < 8000 and 100 < peaks["mfma_bf16_TFLOPs"] < 2500
