"""Benchmark of one Barnes-Hut force evaluation on one MI355X.

A step is one whole evaluation through the C ABI (orr_eval_forces): root cube,
Morton keys, radix sort, gather, tree build, moments, coherent walk and
scatter, with the particles already resident in HBM. The workload is the
Plummer sphere of 1,048,576 particles (softening 0.05, opening angle 0.5, leaf
capacity 32, float32; seed 20260811, generator in
barnes_hut_gravitational_amd/inputs.py).

Prints one JSON line. value = particle-node interactions per second of the
whole evaluation: sum over targets of (particle terms + accepted cells),
divided by the mean step time.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

METRIC = "ms per force eval + particle-node interactions/s, Plummer N=1M, theta 0.5"
FLOPS_PER_INTERACTION = 20       # 3 sub, 6 for r^2 + eps^2, sqrt + div, 3 mul, 6 for a += f d
PEAK_FP32_TFLOPS = 157.3         # MI355X FP32 vector (packed); non-packed issue is half of it
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="plummer_1m")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-trials", type=int, default=3,
                    help="whole oracle evaluations timed for the CPU baseline (median)")
    ap.add_argument("--no-direct", action="store_true",
                    help="skip the all-pairs direct-sum leg (Plummer 131,072)")
    ap.add_argument("--no-accuracy", action="store_true",
                    help="skip the errors against the float64 direct sum (65k whole; 131k, 1M, 8M sampled)")
    ap.add_argument("--no-width-sweep", action="store_true",
                    help="skip the group-width sweep of the walk (orr_tree_walk_grouped)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-workload table (every workload, both traversals)")
    ap.add_argument("--no-scaling", action="store_true",
                    help="skip the Plummer scaling sweep (N = 2^10 .. 2^21)")
    ap.add_argument("--no-shard", action="store_true",
                    help="skip the one-GPU share leg (range walks of the 8M merger split 8 ways)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB first (counter calibration)")
    ap.add_argument("--csv-dir", default=None,
                    help="also write scaling.csv (the Plummer sweep) and divergence.csv (every workload, "
                         "both traversals) into this directory")
    return ap.parse_args()


SCALING_COLUMNS = ("n", "n_nodes", "eval_ms_median", "eval_ms_iqr", "walk_ms_median", "eval_ms_per_n_log2n",
                   "cells_per_particle", "visits_own_per_particle", "visits_stepped_per_particle")
DIVERGENCE_COLUMNS = ("workload", "n", "n_nodes", "eval_ms_median", "eval_ms_iqr", "coherent_walk_ms",
                      "independent_walk_ms", "coherent_speedup_walk", "visits_own_per_particle",
                      "visits_stepped_per_particle", "redundancy", "interactions", "interactions_per_s_walk")


def write_csvs(csv_dir, scaling, configs):
    """The benchmark's two tables as CSV, one row per size or workload (the
    scaling and divergence files of the orrery performance page, "Scaling,
    and where it stops" and "The divergence mitigation")."""
    import csv
    os.makedirs(csv_dir, exist_ok=True)
    written = []
    if scaling:
        path = os.path.join(csv_dir, "scaling.csv")
        with open(path, "w", newline="") as f:
            w = csv.writer(f)
            w.writerow(SCALING_COLUMNS)
            for n, row in sorted(scaling.items(), key=lambda kv: int(kv[0])):
                w.writerow([int(n)] + [row[c] for c in SCALING_COLUMNS[1:]])
        written.append(path)
    if configs:
        path = os.path.join(csv_dir, "divergence.csv")
        with open(path, "w", newline="") as f:
            w = csv.writer(f)
            w.writerow(DIVERGENCE_COLUMNS)
            for name, row in configs.items():
                w.writerow([name, row["n"], row["n_nodes"], row["eval_ms_median"], row["eval_ms_iqr"],
                            row["walk_ms_median"]["coherent"], row["walk_ms_median"]["independent"],
                            row["coherent_speedup_walk"], row["visits_own_per_particle"],
                            row["visits_stepped_per_particle"], row["redundancy"], row["interactions"],
                            row["interactions_per_s_walk"]])
        written.append(path)
    return written


def percentile(v, q):
    v = sorted(v)
    k = (len(v) - 1) * q
    lo = int(k)
    hi = min(lo + 1, len(v) - 1)
    return v[lo] + (v[hi] - v[lo]) * (k - lo)


def walk_traffic_bytes():
    """HBM bytes per coherent-walk launch from the committed rocprofv3 counter
    summary, or None if the walk source has changed since it was taken."""
    import hashlib

    root = os.path.dirname(os.path.abspath(__file__))
    prof = os.path.join(root, "profiles", "k_walk_coherent_plummer_1m.md")
    csrc = os.path.join(root, "barnes_hut_gravitational_amd", "csrc")
    try:
        fields = dict(l.split(": ", 1) for l in open(prof).read().splitlines()[:5] if ": " in l)
        h = hashlib.sha256()
        for name in ("walk.hip", "walk_common.h", "walk_leaf.h", "term.h", "schedule.h", "checked.h"):  # the walk and what it inlines
            h.update(open(os.path.join(csrc, name), "rb").read())
        digest = h.hexdigest()[:16]
        if fields.get("walk-source-sha256-16", "").strip() == digest:
            return int(fields["traffic-bytes-per-launch"])
    except (OSError, KeyError, ValueError):
        pass
    return None


def direct_leg(dev, stream, trials=5, accuracy=True):
    """The all-pairs direct sum (orr_direct_forces) with the walk's term: its
    rate on the Plummer sphere of 131,072 particles (every lane does useful
    work on every term, so this is the issue-bound rate of the exact term
    itself); the tree/direct crossover over Plummer spheres of 2^10 .. 2^17
    particles (the pages' GPU direct column, "Against the two solvers it has
    to beat"); and the tree's error at theta 0.5, and the float32 direct
    sum's, against the compensated float64 direct sum ("Accuracy";
    orr_direct_forces_fp64_targets) on every target of Plummer 65,536 and on
    sampled targets of Plummer 131k, 1M and the 8M merger."""
    import math

    import numpy as np
    import torch
    from barnes_hut_gravitational_amd import inputs, orr

    def timed(run, reps):
        run()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        torch.cuda.synchronize()
        ev[0].record(stream)
        for k in range(reps):
            run()
            ev[k + 1].record(stream)
        torch.cuda.synchronize()
        return percentile([ev[k].elapsed_time(ev[k + 1]) for k in range(reps)], 0.5)

    pos_np, mass_np = inputs.make_config("plummer_131k")
    P, M = torch.from_numpy(pos_np).to(dev), torch.from_numpy(mass_np).to(dev)
    acc = torch.empty((len(mass_np), 3), dtype=torch.float32, device=dev)
    t = timed(lambda: orr.orr_direct_forces(P, M, eps=inputs.EPS, out=acc), trials)
    n = len(mass_np)
    inter = n * (n - 1)
    achieved = FLOPS_PER_INTERACTION * inter / (t * 1e-3) / 1e12
    out = {"workload": "plummer_131k", "kernel": "k_direct", "ms_median": t, "interactions": inter,
           "interactions_per_s": inter / (t * 1e-3), "achieved": achieved, "unit": "TFLOP/s",
           "frac": achieved / PEAK_FP32_TFLOPS}
    # tree (whole evaluation) against direct, N = 2^10 .. 2^17
    rows, prev = {}, None
    crossover = None
    for e in range(10, 18):
        nn = 1 << e
        p_np, m_np = inputs.make("plummer", nn)
        Pn, Mn = torch.from_numpy(p_np).to(dev), torch.from_numpy(m_np).to(dev)
        a = torch.empty((nn, 3), dtype=torch.float32, device=dev)
        ws = orr.new_workspace(nn, inputs.LEAF_CAP, dev)
        cnt = [torch.empty(nn, dtype=torch.int32, device=dev) for _ in range(4)]
        td = timed(lambda: orr.orr_direct_forces(Pn, Mn, eps=inputs.EPS, out=a), trials)
        tt = timed(lambda: orr.orr_eval_forces(Pn, Mn, eps=inputs.EPS, theta=inputs.THETA, leaf_cap=inputs.LEAF_CAP,
                                               workspace=ws, out=(a, cnt)), trials)
        rows[str(nn)] = {"direct_ms": td, "tree_eval_ms": tt, "tree_over_direct": tt / td}
        r = math.log(tt / td)
        if crossover is None and prev is not None and prev[1] > 0 >= r:
            # log-linear interpolation of the tree/direct time ratio between the two sizes
            crossover = math.exp(math.log(prev[0]) + (math.log(nn) - math.log(prev[0])) * prev[1] / (prev[1] - r))
        prev = (nn, r)
        del Pn, Mn, a, ws, cnt
    out["crossover"] = {"rows": rows, "tree_faster_from_n": crossover}
    err = {}

    def summary(got, ref):
        d = (got.double() - ref).norm(dim=1)
        a = ref.norm(dim=1)
        rel = d / a
        return {"rel_rms": float(rel.pow(2).mean().sqrt()), "rel_median": float(rel.median()),
                "rel_p99": float(torch.quantile(rel, 0.99)), "rel_max": float(rel.max()),
                "rms_over_rms": float(d.pow(2).mean().sqrt() / a.pow(2).mean().sqrt())}

    # against the compensated float64 direct sum (the pages' reference) on
    # sampled targets; the float32 direct sum's own error on the same targets
    # beside it (the pages give 3.7e-6 rms for their GPU direct kernel at 65,536)
    samples = {"plummer_65k": ("plummer", 65536, None), "plummer_131k": ("plummer", 131072, 32768),
               "plummer_1m": ("plummer", 1 << 20, 32768), "merger_8m": ("merger", 1 << 23, 16384)}
    for name, (kind, nn, m) in samples.items() if accuracy else ():
        pos_np, mass_np = inputs.make(kind, nn)
        P, M = torch.from_numpy(pos_np).to(dev), torch.from_numpy(mass_np).to(dev)
        tree = orr.orr_eval_forces(P, M, eps=inputs.EPS, theta=inputs.THETA, leaf_cap=inputs.LEAF_CAP).acc
        idx = np.arange(nn) if m is None else np.sort(np.random.default_rng(20260811).choice(nn, m, replace=False))
        ti = torch.from_numpy(idx.astype(np.int64)).to(dev)
        ref = orr.orr_direct_forces_fp64_targets(P, M, ti, eps=inputs.EPS)
        d32 = orr.orr_direct_forces_targets(P, M, ti, eps=inputs.EPS)
        torch.cuda.synchronize()
        err[name] = {"targets": int(len(idx)), "tree_theta_0.5": summary(tree[ti], ref),
                     "direct_fp32": summary(d32, ref)}
        del P, M, tree, ref, d32, ti
        torch.cuda.empty_cache()
    out["error_vs_fp64_direct"] = err or None
    return out


def width_sweep(tree, acc, cnt, stream, trials=4):
    """Walk time and stepped visits per target for groups of W targets sharing
    a node index (orr_tree_walk_grouped, vector loads), W = 1 .. 64, on the
    benchmark's tree: the sub-group width question of the orrery pages."""
    import torch
    from barnes_hut_gravitational_amd import inputs

    out = {}
    for w in (1, 2, 4, 8, 16, 32, 64):
        tree.walk_grouped(inputs.EPS, inputs.THETA, w, out=(acc, cnt))
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(trials + 1)]
        ev[0].record(stream)
        for k in range(trials):
            tree.walk_grouped(inputs.EPS, inputs.THETA, w, out=(acc, cnt))
            ev[k + 1].record(stream)
        torch.cuda.synchronize()
        stepped = cnt[1].to(torch.int64).sum().item() / cnt[1].numel()
        out[str(w)] = {"walk_ms_median": percentile([ev[k].elapsed_time(ev[k + 1]) for k in range(trials)], 0.5),
                       "visits_stepped_per_particle": stepped}
    return out


def production_width_leg(tree, acc, cnt, stream, trials=4):
    """The coherent walk at coherence width 32, 64, 128 and 256 with the
    production machinery (orr_tree_walk_width: scalar node loads, LDS
    leaves; two node indices per wave at 32, work-group coherence at 128 and
    256): walk time and stepped visits per target."""
    import torch
    from barnes_hut_gravitational_amd import inputs

    out = {}
    for w in (32, 64, 128, 256):
        tree.walk_width(inputs.EPS, inputs.THETA, w, out=(acc, cnt))
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(trials + 1)]
        ev[0].record(stream)
        for k in range(trials):
            tree.walk_width(inputs.EPS, inputs.THETA, w, out=(acc, cnt))
            ev[k + 1].record(stream)
        torch.cuda.synchronize()
        stepped = cnt[1].to(torch.int64).sum().item() / cnt[1].numel()
        out[str(w)] = {"walk_ms_median": percentile([ev[k].elapsed_time(ev[k + 1]) for k in range(trials)], 0.5),
                       "visits_stepped_per_particle": stepped}
    return out


def descend_leg(tree, acc, cnt, stream, trials=4):
    """The descend-together group walk (orr_tree_walk_descend: a group opens a
    node when any member would, all members descending), for comparison with
    the masked walk at the same group width."""
    import torch
    from barnes_hut_gravitational_amd import inputs

    out = {}
    for w in (32, 64):
        tree.walk_descend(inputs.EPS, inputs.THETA, w, out=(acc, cnt))
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(trials + 1)]
        ev[0].record(stream)
        for k in range(trials):
            tree.walk_descend(inputs.EPS, inputs.THETA, w, out=(acc, cnt))
            ev[k + 1].record(stream)
        torch.cuda.synchronize()
        inter = int(cnt[2].long().sum().item() + cnt[3].long().sum().item())
        out[str(w)] = {"walk_ms_median": percentile([ev[k].elapsed_time(ev[k + 1]) for k in range(trials)], 0.5),
                       "interactions": inter}
    return out


def advance_leg(tree, acc, cnt, stream, trials=6):
    """Cost of the wave advance rule: the coherent walk (select between c + 1
    and the escape on the mask of opening lanes) against the same walk taking
    an explicit DPP minimum of the lanes' next nodes at every step
    (orr_tree_walk_min_advance); both visit the same nodes."""
    import torch
    from barnes_hut_gravitational_amd import inputs

    runs = {"mask_select": lambda: tree.walk(inputs.EPS, inputs.THETA, traversal="coherent", out=(acc, cnt)),
            "dpp_min": lambda: tree.walk_min_advance(inputs.EPS, inputs.THETA, out=(acc, cnt))}
    out = {}
    for name, run in runs.items():
        run()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(trials + 1)]
        ev[0].record(stream)
        for k in range(trials):
            run()
            ev[k + 1].record(stream)
        torch.cuda.synchronize()
        out[name] = {"walk_ms_median": percentile([ev[k].elapsed_time(ev[k + 1]) for k in range(trials)], 0.5)}
    return out


def shard_leg(dev, stream, k=8, trials=4, workload="merger_8m"):
    """One GPU's share of the 8M merger's targets: the sorted targets split
    into k contiguous ranges of whole waves, by the estimated walk cost
    (orr_tree_shard_bounds) and, for comparison, by count; each range walked
    alone with the coherent walk (orr_tree_walk_range), as each of k GPUs
    would walk its share of the same tree. The slowest range bounds the time
    k GPUs would take for the walk."""
    import torch
    from barnes_hut_gravitational_amd import inputs, orr

    kind, n = inputs.CONFIGS[workload]
    pos_np, mass_np = inputs.make(kind, n)
    pos = torch.from_numpy(pos_np).to(dev)
    mass = torch.from_numpy(mass_np).to(dev)
    tree = orr.Tree(pos, mass, inputs.LEAF_CAP)
    acc = torch.empty((n, 3), dtype=torch.float32, device=dev)
    cnt = [torch.empty(n, dtype=torch.int32, device=dev) for _ in range(4)]
    perm = tree.export()["perm"].long()

    def timed(run):
        run()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(trials + 1)]
        ev[0].record(stream)
        for j in range(trials):
            run()
            ev[j + 1].record(stream)
        torch.cuda.synchronize()
        return percentile([ev[j].elapsed_time(ev[j + 1]) for j in range(trials)], 0.5)

    whole = timed(lambda: tree.walk(inputs.EPS, inputs.THETA, "coherent", out=(acc, cnt)))
    work = (cnt[2].long() + cnt[3].long())[perm]  # interactions per sorted target
    nw = (n + 63) // 64
    splits = {"estimated_cost": tree.shard_bounds(k),
              "equal_count": [min(64 * ((nw * j) // k), n) for j in range(k + 1)]}
    out = {"workload": workload, "n": n, "k": k, "whole_walk_ms": whole}
    for name, b in splits.items():
        ms, inter = [], []
        for a, z in zip(b, b[1:]):
            ms.append(timed(lambda: tree.walk_range(a, z - a, inputs.EPS, inputs.THETA, "coherent",
                                                    out=(acc, cnt))))
            inter.append(int(work[a:z].sum().item()))
        out[name] = {"bounds": b, "range_ms": ms, "max_ms": max(ms), "sum_ms": sum(ms),
                     "interactions": inter, "max_over_mean_interactions": max(inter) * k / sum(inter)}
    del tree
    torch.cuda.empty_cache()
    return out


def configs_leg(dev, stream, trials=11, walk_trials=5):
    """Every workload: whole evaluations (median and IQR of `trials`), the
    walk alone with both traversals, interactions and node visits per
    particle."""
    import torch

    from barnes_hut_gravitational_amd import inputs, orr

    table = {}
    for name, (kind, n) in inputs.CONFIGS.items():
        pos_np, mass_np = inputs.make(kind, n)
        pos = torch.from_numpy(pos_np).to(dev)
        mass = torch.from_numpy(mass_np).to(dev)
        ws = orr.new_workspace(n, inputs.LEAF_CAP, dev)
        acc = torch.empty((n, 3), dtype=torch.float32, device=dev)
        cnt = [torch.empty(n, dtype=torch.int32, device=dev) for _ in range(4)]
        kw = dict(eps=inputs.EPS, theta=inputs.THETA, leaf_cap=inputs.LEAF_CAP, workspace=ws, out=(acc, cnt))
        for _ in range(2):
            orr.orr_eval_forces(pos, mass, traversal="coherent", **kw)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(trials + 1)]
        torch.cuda.synchronize()
        ev[0].record(stream)
        for k in range(trials):
            orr.orr_eval_forces(pos, mass, traversal="coherent", **kw)
            ev[k + 1].record(stream)
        torch.cuda.synchronize()
        full = [ev[k].elapsed_time(ev[k + 1]) for k in range(trials)]
        inter = int(cnt[2].long().sum().item() + cnt[3].long().sum().item())
        own = float(cnt[0].double().mean().item())
        stepped = float(cnt[1].double().mean().item())
        pp_mean = float(cnt[2].double().mean().item())
        pc_mean = float(cnt[3].double().mean().item())
        tree = orr.Tree(pos, mass, inputs.LEAF_CAP, workspace=ws)
        walk = {}
        for tr in ("coherent", "independent"):
            tree.walk(inputs.EPS, inputs.THETA, tr, out=(acc, cnt))
            wev = [torch.cuda.Event(enable_timing=True) for _ in range(walk_trials + 1)]
            wev[0].record(stream)
            for k in range(walk_trials):
                tree.walk(inputs.EPS, inputs.THETA, tr, out=(acc, cnt))
                wev[k + 1].record(stream)
            torch.cuda.synchronize()
            walk[tr] = percentile([wev[k].elapsed_time(wev[k + 1]) for k in range(walk_trials)], 0.5)
        row = {"n": n, "eval_ms_median": percentile(full, 0.5),
               "eval_ms_iqr": percentile(full, 0.75) - percentile(full, 0.25),
               "walk_ms_median": walk, "coherent_speedup_walk": walk["independent"] / walk["coherent"],
               "interactions": inter, "interactions_per_s_eval": inter / (percentile(full, 0.5) * 1e-3),
               "interactions_per_s_walk": inter / (walk["coherent"] * 1e-3),
               "visits_own_per_particle": own, "visits_stepped_per_particle": stepped,
               "redundancy": stepped / own, "particle_terms_per_particle": pp_mean,
               "cells_per_particle": pc_mean, "n_nodes": tree.info()["n_nodes"]}
        table[name] = row
        del tree, ws, acc, cnt, pos, mass
        torch.cuda.empty_cache()
    return table


def scaling_leg(dev, stream, trials=11):
    """Plummer spheres of N = 2^10 .. 2^21 (the sizes of the pages' scaling
    table): whole evaluation and walk medians, per-particle counts, and the
    evaluation time over N log2 N."""
    import math

    import torch

    from barnes_hut_gravitational_amd import inputs, orr

    rows = {}
    for e in range(10, 22):
        n = 1 << e
        pos_np, mass_np = inputs.make("plummer", n)
        pos = torch.from_numpy(pos_np).to(dev)
        mass = torch.from_numpy(mass_np).to(dev)
        ws = orr.new_workspace(n, inputs.LEAF_CAP, dev)
        acc = torch.empty((n, 3), dtype=torch.float32, device=dev)
        cnt = [torch.empty(n, dtype=torch.int32, device=dev) for _ in range(4)]
        kw = dict(eps=inputs.EPS, theta=inputs.THETA, leaf_cap=inputs.LEAF_CAP, workspace=ws, out=(acc, cnt))
        tree = orr.Tree(pos, mass, inputs.LEAF_CAP, workspace=ws)
        times = {}
        for name, run in (("eval", lambda: orr.orr_eval_forces(pos, mass, traversal="coherent", **kw)),
                          ("walk", lambda: tree.walk(inputs.EPS, inputs.THETA, "coherent", out=(acc, cnt)))):
            run()
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(trials + 1)]
            torch.cuda.synchronize()
            ev[0].record(stream)
            for k in range(trials):
                run()
                ev[k + 1].record(stream)
            torch.cuda.synchronize()
            ts = [ev[k].elapsed_time(ev[k + 1]) for k in range(trials)]
            times[name] = (percentile(ts, 0.5), percentile(ts, 0.75) - percentile(ts, 0.25))
        rows[str(n)] = {"eval_ms_median": times["eval"][0], "eval_ms_iqr": times["eval"][1],
                        "walk_ms_median": times["walk"][0],
                        "eval_ms_per_n_log2n": times["eval"][0] / (n * math.log2(n)),
                        "cells_per_particle": float(cnt[3].double().mean().item()),
                        "visits_own_per_particle": float(cnt[0].double().mean().item()),
                        "visits_stepped_per_particle": float(cnt[1].double().mean().item()),
                        "n_nodes": tree.info()["n_nodes"]}
        del tree, ws, acc, cnt, pos, mass
        torch.cuda.empty_cache()
    return rows


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(pos, mass, trials):
    """The oracle as it stands, on this host's cores: whole evaluations of the
    workload (build, walk of every target, group union visits), median; then
    every other workload (Plummer 16k, 131k, uniform 262k: 11 evaluations on
    all threads, and Plummer 16k and 131k 3 on one thread; the 8M merger once
    on all threads)."""
    import numpy as np

    import oracle
    from barnes_hut_gravitational_amd import inputs

    def timed(p, m, reps):
        ts, inter = [], 0
        for _ in range(reps):
            t0 = time.perf_counter()
            r = oracle.evaluate(p, m, inputs.EPS, inputs.THETA, inputs.LEAF_CAP)
            ts.append(time.perf_counter() - t0)
            inter = int(r.n_pp.sum(dtype=np.int64) + r.n_pc.sum(dtype=np.int64))
        return ts, inter

    times, inter = timed(pos, mass, trials)
    med = percentile(times, 0.5)
    all_threads = oracle.num_threads()
    per_config = {}
    plan = [("plummer_16k", all_threads, 11), ("plummer_131k", all_threads, 11), ("uniform_262k", all_threads, 11),
            ("plummer_16k", 1, 3), ("plummer_131k", 1, 3), ("merger_8m", all_threads, 1)]
    for name, threads, reps in plan:
        kind, n = inputs.CONFIGS[name]
        p, m = inputs.make(kind, n)
        oracle.set_num_threads(threads)
        ts, k = timed(p, m, reps)
        oracle.set_num_threads(all_threads)
        row = per_config.setdefault(name, {})
        row[str(threads)] = {"eval_ms_median": percentile(ts, 0.5) * 1e3,
                             "eval_ms_iqr": (percentile(ts, 0.75) - percentile(ts, 0.25)) * 1e3, "trials": reps,
                             "interactions_per_s": k / percentile(ts, 0.5)}
        del p, m
    return {"value": inter / med, "unit": "interactions/s", "cores": all_threads, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"{trials} whole oracle evaluations of the workload (tree build serial; walk and group "
                      f"union visits OpenMP over targets on {all_threads} threads), median {med * 1e3:.0f} ms, "
                      f"total {sum(times):.1f} s; then the other workloads (per_config)",
            "eval_ms": med * 1e3, "eval_ms_iqr": (percentile(times, 0.75) - percentile(times, 0.25)) * 1e3,
            "per_config_eval_ms_by_threads": per_config}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (run with --gpus 1).",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from barnes_hut_gravitational_amd import inputs, orr

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    orr.lib()
    kind, n = inputs.CONFIGS[args.workload]
    pos_np, mass_np = inputs.make(kind, n)
    dev = torch.device("cuda:0")
    pos = torch.from_numpy(pos_np).to(dev)
    mass = torch.from_numpy(mass_np).to(dev)
    ws = orr.new_workspace(n, inputs.LEAF_CAP, dev)
    acc = torch.empty((n, 3), dtype=torch.float32, device=dev)
    cnt = [torch.empty(n, dtype=torch.int32, device=dev) for _ in range(4)]
    kw = dict(eps=inputs.EPS, theta=inputs.THETA, leaf_cap=inputs.LEAF_CAP, workspace=ws, out=(acc, cnt))
    stream = torch.cuda.current_stream(dev)

    def step(traversal="coherent"):
        orr.orr_eval_forces(pos, mass, traversal=traversal, **kw)

    if args.copy_mib:
        # a plain copy of known size: HBM traffic counters are scaled by what they read for it
        src = torch.empty(args.copy_mib << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for _ in range(args.warmup):
        step()
    orr.orr_workspace_check(ws)  # raises on non-finite input or an invalid sort
    # counts of the workload (identical every step)
    inter = int(cnt[2].long().sum().item() + cnt[3].long().sum().item())
    visits_own = float(cnt[0].double().mean().item())
    visits_stepped = float(cnt[1].double().mean().item())

    # timed region: K whole evaluations, events per step on the library's stream
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev[0].record(stream)
    for k in range(args.steps):
        step()
        ev[k + 1].record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    step_ms = [ev[k].elapsed_time(ev[k + 1]) for k in range(args.steps)]
    # the last timed evaluation: valid input and sort, and the warm-up's counts
    orr.orr_workspace_check(ws)
    if int(cnt[2].long().sum().item() + cnt[3].long().sum().item()) != inter:
        raise RuntimeError("the timed evaluations' interaction count differs from the warm-up's")

    # the dominant kernel alone: K walks of the built tree, both traversals
    tree = orr.Tree(pos, mass, inputs.LEAF_CAP, workspace=ws)
    walk_ms = {}
    for tr in ("coherent", "independent"):
        tree.walk(inputs.EPS, inputs.THETA, tr, out=(acc, cnt))
        wev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        wev[0].record(stream)
        for k in range(args.steps):
            tree.walk(inputs.EPS, inputs.THETA, tr, out=(acc, cnt))
            wev[k + 1].record(stream)
        torch.cuda.synchronize()
        walk_ms[tr] = [wev[k].elapsed_time(wev[k + 1]) for k in range(args.steps)]
    phases = orr.orr_eval_forces(pos, mass, traversal="coherent", timings=True, **kw).timings
    info = tree.info()
    direct = None if args.no_direct else direct_leg(dev, stream, accuracy=not args.no_accuracy)
    widths = None if args.no_width_sweep else width_sweep(tree, acc, cnt, stream)
    prod_widths = None if args.no_width_sweep else production_width_leg(tree, acc, cnt, stream)
    descend = None if args.no_width_sweep else descend_leg(tree, acc, cnt, stream)
    advance = None if args.no_width_sweep else advance_leg(tree, acc, cnt, stream)
    shard = None if args.no_shard else shard_leg(dev, stream)
    configs = None if args.no_configs else configs_leg(dev, stream)
    scaling = None if args.no_scaling else scaling_leg(dev, stream)

    ms = wall_ms
    walk_mean = sum(walk_ms["coherent"]) / args.steps
    achieved = FLOPS_PER_INTERACTION * inter / (walk_mean * 1e-3) / 1e12
    traffic = walk_traffic_bytes() if args.workload == "plummer_1m" else None
    out = {
        "metric": METRIC,
        "value": inter / (ms * 1e-3),
        "unit": "interactions/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": args.workload, "kind": kind, "n": n, "eps": inputs.EPS, "theta": inputs.THETA,
                   "leaf_cap": inputs.LEAF_CAP, "traversal": "coherent", "seed": inputs.SEED},
        "roofline": {"bound": "alu", "kernel": "k_walk_coherent", "achieved": achieved, "peak": PEAK_FP32_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / PEAK_FP32_TFLOPS,
                     "frac_of_unpacked_peak": achieved / (PEAK_FP32_TFLOPS / 2),
                     "traffic": traffic,
                     "hbm_gbs": traffic / (walk_mean * 1e-3) / 1e9 if traffic else None,
                     "hbm_frac": traffic / (walk_mean * 1e-3) / 1e9 / PEAK_HBM_GBS if traffic else None,
                     "flops_per_interaction": FLOPS_PER_INTERACTION, "walk_ms_mean": walk_mean},
        "step_ms_median": percentile(step_ms, 0.5),
        "step_ms_iqr": percentile(step_ms, 0.75) - percentile(step_ms, 0.25),
        "walk_ms_median": {k: percentile(v, 0.5) for k, v in walk_ms.items()},
        "coherent_speedup_walk": percentile(walk_ms["independent"], 0.5) / percentile(walk_ms["coherent"], 0.5),
        "walk_interactions_per_s": inter / (walk_mean * 1e-3),
        "interactions": inter,
        "visits_own_per_particle": visits_own,
        "visits_stepped_per_particle": visits_stepped,
        "redundancy": visits_stepped / visits_own,
        "phases_ms": phases,
        "tree": {"n_nodes": info["n_nodes"], "depth": info["depth"], "n_leaves": info["n_leaves"]},
        "direct": direct,
        "width_sweep": widths,
        "production_widths": prod_widths,
        "descend_together": descend,
        "advance_rule": advance,
        "one_gpu_share": shard,
        "configs": configs,
        "scaling_sweep": scaling,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(pos_np, mass_np, args.cpu_trials)
    if args.csv_dir:
        for path in write_csvs(args.csv_dir, scaling, configs):
            print(f"wrote {path}", file=sys.stderr, flush=True)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
