"""The checked build (liborr_checked.so, device index checks) on the GPU, run
by test_gpu_checked.py in a process of its own with ORR_CHECKED=1 (the binding
loads one library per process).

1. Clean inputs: every entry point's results equal the oracle's (or the
   normal build's contract) bit for bit, and no check fires (each
   synchronising call returns ORR_OK).
2. A corrupted tree: the last node record's particle count is raised by one,
   so its leaf range ends one past the particles. The walks' leaf check must
   fire, skip that leaf, and make the next synchronising call fail with
   ORR_ERR_HIP. The range still ends inside the workspace, so even an access
   the check failed to stop would not leave the allocation.

Prints one line per case and "checked driver ok" at the end.
"""

import os
import sys

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))
sys.path.insert(0, HERE)

import oracle  # noqa: E402
from barnes_hut_gravitational_amd import inputs, orr  # noqa: E402
from parity import check_acc_bitwise, check_tree, check_walk, to_dev  # noqa: E402


def clustered(n_clusters, per, side, seed):
    rng = np.random.default_rng(seed)
    c = rng.uniform(0.1, 0.9, (n_clusters, 1, 3))
    pos = (c + rng.uniform(0, side, (n_clusters, per, 3))).reshape(-1, 3).astype(np.float32)
    return pos, np.full(len(pos), 1 / len(pos), np.float32)


def clean_case(name, pos, mass, cap, eps=inputs.EPS, theta=inputs.THETA):
    print(f"[checked] {name} n={len(mass)} cap={cap}", flush=True)
    ref = oracle.evaluate(pos, mass, eps, theta, cap)
    P, M = to_dev(pos, mass)
    tree = orr.Tree(P, M, cap)
    check_tree(tree, ref.tree)
    for tr in ("coherent", "independent"):
        r = tree.walk(eps, theta, tr, timings=True)
        check_walk(r, ref, tr)
        check_acc_bitwise(r, ref.acc)
    c = tree.walk(eps, theta, "coherent")
    for w in (32, 128, 256):
        r = tree.walk_width(eps, theta, w)
        torch.cuda.synchronize()
        assert torch.equal(r.acc.view(torch.int32), c.acc.view(torch.int32)), w
    for g in (1, 16):
        r = tree.walk_grouped(eps, theta, g)
        torch.cuda.synchronize()
        assert torch.equal(r.acc.view(torch.int32), c.acc.view(torch.int32)), g
    n = len(mass)
    if n > 128:
        first = 64 * ((n // 64) // 2)
        r = tree.walk_range(first, n - first, eps, theta)
        torch.cuda.synchronize()
    tree.check()
    e = orr.orr_eval_forces(P, M, eps=eps, theta=theta, leaf_cap=cap, timings=True)
    check_acc_bitwise(e, ref.acc)


def corrupted_leaf():
    n, cap = 5000, 16
    pos, mass = inputs.make("plummer", n)
    print(f"[checked] corrupted last leaf n={n} cap={cap}", flush=True)
    P, M = to_dev(pos, mass)
    ws = orr.new_workspace(n, cap, P.device)
    tree = orr.Tree(P, M, cap, workspace=ws)
    tree.check()
    ex = tree.export()
    esc, beg, cnt = (t.cpu().numpy().view(np.uint32) for t in (ex["escape"], ex["begin"], ex["count"]))
    s2 = ex["s2"].cpu().numpy().view(np.uint32)
    last = len(esc) - 1
    assert esc[last] == last + 1 and beg[last] + cnt[last] == n  # the last node is a leaf ending at n
    # The record's second half (escape, begin, count, s^2 bits) in the workspace.
    w = ws.cpu().numpy().view(np.uint32)
    pat = np.array([esc[last], beg[last], cnt[last], s2[last]], np.uint32)
    cand = np.flatnonzero(w[:-3] == pat[0])
    hits = [int(p) for p in cand if np.array_equal(w[p:p + 4], pat)]
    assert len(hits) == 1, hits
    words = ws.view(torch.int32)
    words[hits[0] + 2] += 1
    # The workspace starts with the build's device parameters; word 5 is the
    # status word (bit 2: an index check failed). It stays set until the next
    # build, so it is cleared before each walk to see that walk's own report.
    status = 5
    assert int(words[status]) == 0
    for tr in ("coherent", "independent"):
        words[status] = 0
        torch.cuda.synchronize()
        tree.check()
        tree.walk(inputs.EPS, inputs.THETA, tr)
        torch.cuda.synchronize()
        assert int(words[status]) == 4, int(words[status])
        try:
            tree.check()
        except orr.OrrError as e:
            assert e.status == orr.ORR_ERR_HIP and "index check" in str(e), str(e)
            print(f"[checked] {tr} walk reported: {e}", flush=True)
        else:
            raise AssertionError(f"the {tr} walk's leaf check did not fire")


def main():
    assert os.environ.get("ORR_CHECKED") == "1" and orr.LIB_PATH.endswith("liborr_checked.so")
    assert torch.cuda.is_available()
    orr.lib()
    for kind, n, cap in (("plummer", 5000, 16), ("plummer", 20000, 32), ("merger", 70000, 8), ("uniform", 3000, 1)):
        pos, mass = inputs.make(kind, n)
        clean_case(f"{kind}", pos, mass, cap)
    rng = np.random.default_rng(3)
    lat = rng.integers(0, 3, (3000, 3)).astype(np.float32)
    clean_case("lattice", lat, np.full(3000, 1 / 3000, np.float32), 8)
    pos, mass = clustered(3, 30000, 1e-5, 41)  # runs longer than 4,096: the fallback's runs mode
    clean_case("clusters-3", pos, mass, 32)
    pos, mass = clustered(70, 5000, 1e-6, 43)  # more than 64 long runs: the fallback's full mode
    clean_case("clusters-70", pos, mass, 32)
    corrupted_leaf()
    print("checked driver ok", flush=True)


if __name__ == "__main__":
    main()
