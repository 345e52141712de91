"""CPU-side checks of the benchmark's command-line contract: more than one GPU
is refused with a message (this build measures one GPU), and the JSON line's
helpers behave. No GPU is touched."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args, env=None):
    e = dict(os.environ)
    e.update(env or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          cwd=ROOT, env=e, timeout=120)


@pytest.mark.parametrize("args,env", [(("--gpus", "2"), None), (("--gpus", "8"), None),
                                      ((), {"WORLD_SIZE": "4"})])
def test_more_than_one_gpu_is_refused(args, env):
    r = run_bench(*args, env=env)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_percentile_and_traffic_helpers():
    sys.path.insert(0, ROOT)
    import bench

    assert bench.percentile([3.0, 1.0, 2.0], 0.5) == 2.0
    assert bench.percentile([1.0, 2.0, 3.0, 4.0], 0.0) == 1.0
    assert bench.percentile([1.0, 2.0, 3.0, 4.0], 1.0) == 4.0
    t = bench.walk_traffic_bytes()
    assert t is None or (isinstance(t, int) and t > 0)


def test_profile_header_names_its_hash():
    # the committed walk profile carries the hash bench.py compares with
    with open(os.path.join(ROOT, "profiles", "k_walk_coherent_plummer_1m.md")) as f:
        head = [next(f) for _ in range(5)]
    keys = [l.split(": ", 1)[0] for l in head if ": " in l]
    assert "walk-source-sha256-16" in keys and "traffic-bytes-per-launch" in keys
