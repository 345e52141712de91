"""CPU-side checks of the benchmark's command-line contract: more than one GPU
is refused with a message (the benchmark measures one GPU), and the JSON line's
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


def test_csv_tables(tmp_path):
    sys.path.insert(0, ROOT)
    import csv

    import bench

    scaling = {"2048": {"n_nodes": 334, "eval_ms_median": 0.34, "eval_ms_iqr": 0.002, "walk_ms_median": 0.23,
                        "eval_ms_per_n_log2n": 1.5e-5, "cells_per_particle": 134.0,
                        "visits_own_per_particle": 259.0, "visits_stepped_per_particle": 315.0},
               "1024": {"n_nodes": 165, "eval_ms_median": 0.23, "eval_ms_iqr": 0.001, "walk_ms_median": 0.13,
                        "eval_ms_per_n_log2n": 2.2e-5, "cells_per_particle": 60.0,
                        "visits_own_per_particle": 142.0, "visits_stepped_per_particle": 163.0}}
    configs = {"plummer_16k": {"n": 16384, "n_nodes": 2160, "eval_ms_median": 0.6, "eval_ms_iqr": 0.01,
                               "walk_ms_median": {"coherent": 0.48, "independent": 5.6},
                               "coherent_speedup_walk": 11.7, "visits_own_per_particle": 776.0,
                               "visits_stepped_per_particle": 1098.0, "redundancy": 1.415,
                               "interactions": 31028287, "interactions_per_s_walk": 6.5e10}}
    paths = bench.write_csvs(str(tmp_path), scaling, configs)
    assert [os.path.basename(p) for p in paths] == ["scaling.csv", "divergence.csv"]
    rows = list(csv.reader(open(paths[0])))
    assert tuple(rows[0]) == bench.SCALING_COLUMNS
    assert [r[0] for r in rows[1:]] == ["1024", "2048"]  # ascending N
    assert float(rows[1][bench.SCALING_COLUMNS.index("visits_stepped_per_particle")]) == 163.0
    rows = list(csv.reader(open(paths[1])))
    assert tuple(rows[0]) == bench.DIVERGENCE_COLUMNS
    assert rows[1][0] == "plummer_16k" and float(rows[1][bench.DIVERGENCE_COLUMNS.index("independent_walk_ms")]) == 5.6
    assert bench.write_csvs(str(tmp_path / "none"), {}, {}) == []
