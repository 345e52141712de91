"""A seeded sweep over sizes, particle distributions, leaf capacities, opening
angles and softenings, each case against the CPU oracle.

The walk shares one 64-target wave's work among 1 to 16 hardware waves
depending on how many target waves there are, and the sort finishes runs of
equal high key bits in three ways depending on their length. The fixed cases
elsewhere pin the limits of each class; this sweep draws sizes across all of
them (one particle to 600,000) with the other parameters drawn
independently, so that no combination is left to a single hand-picked case.

Each case: the tree bit for bit, both traversals' accelerations bit for bit
and their counts exactly, and the benchmark's entry point (orr_eval_forces,
coherent) equal to the tree walk.
"""

import os

import numpy as np
import pytest
import torch

import oracle
from barnes_hut_gravitational_amd import inputs, orr

from parity import check_acc_bitwise, check_tree, check_walk, to_dev

pytestmark = pytest.mark.gpu

KINDS = ("plummer", "uniform", "merger", "clusters", "lattice")
CAPS = (1, 2, 3, 8, 16, 32, 64, 100, 256)
THETAS = (0.0, 0.2, 0.5, 0.7, 1.0, 1.5)
EPSES = (1e-3, 0.01, 0.05, 0.2)
# ORR_SWEEP_CASES draws more cases (the case i is the same for every count).
N_CASES = int(os.environ.get("ORR_SWEEP_CASES", "80"))
N_MAX = 600000


def draw_case(i):
    """Case i of the sweep: (kind, n, cap, theta, eps, seed). Sizes are
    log-uniform in [1, N_MAX]; an opening angle of 0 (every pair direct) is
    kept to n <= 4000 so the oracle finishes in seconds."""
    rng = np.random.default_rng(7000 + i)
    kind = KINDS[rng.integers(len(KINDS))]
    n = int(np.exp(rng.uniform(0.0, np.log(N_MAX))))
    cap = int(CAPS[rng.integers(len(CAPS))])
    theta = float(THETAS[rng.integers(len(THETAS))])
    if theta == 0.0 and n > 4000:
        theta = 0.5
    eps = float(EPSES[rng.integers(len(EPSES))])
    return kind, n, cap, theta, eps, 100 + i


def particles(kind, n, seed):
    """Positions and masses of one case. clusters: a few tight cubes (runs of
    equal high key bits of every length, longer than 4,096 for the larger
    sizes); lattice: points on a grid of 2^3 to 9^3 (many coincident
    points, over-full leaves at the deepest level). Masses vary per
    particle, some zero."""
    rng = np.random.default_rng(seed)
    if kind in ("plummer", "uniform", "merger"):
        pos, _ = inputs.make(kind, n, seed)
    elif kind == "clusters":
        k = int(rng.integers(1, 6))
        c = rng.uniform(0.1, 0.9, (k, 3))
        side = 10.0 ** rng.uniform(-7, -2)
        pos = (c[rng.integers(0, k, n)] + rng.uniform(0, side, (n, 3))).astype(np.float32)
    else:
        g = int((2, 3, 5, 9)[rng.integers(4)])
        pos = rng.integers(0, g, (n, 3)).astype(np.float32)
    mass = (rng.uniform(0.2, 2.0, n) / n).astype(np.float32)
    mass[rng.random(n) < 0.05] = 0.0
    return np.ascontiguousarray(pos, np.float32), mass


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    orr.lib()


@pytest.mark.parametrize("i", range(N_CASES))
def test_sweep(i):
    kind, n, cap, theta, eps, seed = draw_case(i)
    print(f"[sweep {i}] {kind} n={n} cap={cap} theta={theta} eps={eps} waves={(n + 63) // 64}", flush=True)
    pos, mass = particles(kind, n, seed)
    ref = oracle.evaluate(pos, mass, eps, theta, cap)
    P, M = to_dev(pos, mass)
    tree = orr.Tree(P, M, cap)
    check_tree(tree, ref.tree)
    res = {}
    for tr in ("coherent", "independent"):
        r = tree.walk(eps, theta, tr)
        torch.cuda.synchronize()
        check_walk(r, ref, tr)
        check_acc_bitwise(r, ref.acc)
        res[tr] = r
    for f in ("visits_own", "n_pp", "n_pc"):
        assert torch.equal(getattr(res["coherent"], f), getattr(res["independent"], f))
    e = orr.orr_eval_forces(P, M, eps=eps, theta=theta, leaf_cap=cap, traversal="coherent")
    torch.cuda.synchronize()
    c = res["coherent"]
    assert torch.equal(e.acc.view(torch.int32), c.acc.view(torch.int32))
    for f in ("visits_own", "visits_stepped", "n_pp", "n_pc"):
        assert torch.equal(getattr(e, f), getattr(c, f))
