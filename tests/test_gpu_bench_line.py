"""The benchmark's JSON line from a real run on the GPU (short: 3 timed steps,
the optional legs off, one oracle evaluation for the CPU baseline): every
field of the line's contract is present with the right type, the numbers
agree with each other, and the roofline and CPU-baseline objects are
filled."""

import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_line_contract():
    print("[case] bench.py short run", flush=True)
    cmd = [sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "3", "--warmup", "1", "--cpu-trials", "1",
           "--no-direct", "--no-width-sweep", "--no-configs", "--no-scaling", "--no-shard"]
    r = subprocess.run(cmd, capture_output=True, text=True, cwd=ROOT, timeout=110)
    assert r.returncode == 0, r.stderr[-3000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    d = json.loads(lines[-1])
    print({k: d[k] for k in ("value", "ms_per_step", "steps", "warmup")}, flush=True)

    assert d["unit"] == "interactions/s" and d["higher_is_better"] is True
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["scaling"] == "weak" and d["vs_baseline"] is None
    assert d["dtype"] == "f32" and d["data"] == "synthetic"
    assert d["config"]["workload"] == "plummer_1m" and d["config"]["n"] == 1 << 20
    assert "model" not in d["config"]
    # value is the whole evaluation's rate: interactions over the mean step
    assert d["value"] > 0 and d["ms_per_step"] > 0
    assert abs(d["value"] - d["interactions"] / (d["ms_per_step"] * 1e-3)) <= 1e-6 * d["value"]

    rf = d["roofline"]
    assert rf["bound"] in ("alu", "hbm", "mfma") and rf["unit"] == "TFLOP/s" and rf["peak"] == 157.3
    assert rf["achieved"] > 0 and abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-12
    # achieved = 20 flops per interaction over the walk's mean launch time
    assert abs(rf["achieved"] - 20 * d["interactions"] / (rf["walk_ms_mean"] * 1e-3) / 1e12) <= 1e-9 * rf["achieved"]
    assert rf["traffic"] is None or rf["traffic"] > 0

    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["unit"] == "interactions/s"
    assert cb["value"] > 0 and cb["cores"] >= 1 and isinstance(cb["sample"], str) and cb["sample"]
