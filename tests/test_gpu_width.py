"""GPU parity of the coherent walk at coherence widths 32, 64, 128 and 256
with the production walk's machinery (orr_tree_walk_width): two node indices
per wave at width 32, the production walk at 64, and 2 or 4 waves of a
work-group sharing one node index at 128 and 256. Every target still sums
exactly its own walk, so accelerations and own counts equal the oracle's bit
for bit at every width; visits_stepped equals the size of the union of the
walks of the target's group of `width` consecutive sorted targets, computed
by the oracle for the same grouping."""

import numpy as np
import pytest
import torch

import oracle
from barnes_hut_gravitational_amd import inputs, orr

from parity import to_dev, u32

pytestmark = pytest.mark.gpu
EPS, THETA = inputs.EPS, inputs.THETA
WIDTHS = (32, 64, 128, 256)


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    orr.lib()


def union_caller_order(ot, width, eps, theta):
    u = oracle.union_visits(ot, eps, theta, width)
    out = np.empty(ot.n, np.uint32)
    out[ot.perm] = np.repeat(u, width)[:ot.n]
    return out


def check_widths(pos, mass, cap, theta=THETA, widths=WIDTHS):
    ref = oracle.evaluate(pos, mass, EPS, theta, cap)
    assert np.isfinite(ref.acc).all()
    P, M = to_dev(pos, mass)
    tree = orr.Tree(P, M, cap)
    for w in widths:
        print(f"[case] width walk n={len(mass)} cap={cap} theta={theta} width={w}", flush=True)
        r = tree.walk_width(EPS, theta, w)
        torch.cuda.synchronize()
        assert np.array_equal(r.acc.cpu().numpy().view(np.uint32), ref.acc.view(np.uint32))
        assert np.array_equal(u32(r.visits_own), ref.visits_own)
        assert np.array_equal(u32(r.n_pp), ref.n_pp)
        assert np.array_equal(u32(r.n_pc), ref.n_pc)
        assert np.array_equal(u32(r.visits_stepped), union_caller_order(ref.tree, w, EPS, theta))


@pytest.mark.parametrize("kind,n,cap,theta", [
    ("plummer", 1, 32, THETA), ("plummer", 33, 8, THETA), ("plummer", 100, 32, THETA),
    ("plummer", 4097, 32, THETA), ("merger", 5000, 16, 0.7), ("uniform", 6000, 32, 0.3),
    ("plummer", 3000, 8, 0.25), ("merger", 2048, 3, 100.0), ("plummer", 2000, 8, 0.0)])
def test_widths_small(kind, n, cap, theta):
    pos, mass = inputs.make(kind, n)
    check_widths(pos, mass, cap, theta)


@pytest.mark.parametrize("name", ["plummer_16k", "plummer_131k"])
def test_widths_configs(name):
    pos, mass = inputs.make_config(name)
    check_widths(pos, mass, inputs.LEAF_CAP)


def test_width_rejected():
    P, M = to_dev(*inputs.make("plummer", 100))
    tree = orr.Tree(P, M, 32)
    for w in (0, 16, 48, 512):
        with pytest.raises(orr.OrrError) as e:
            tree.walk_width(EPS, THETA, w)
        assert e.value.status == orr.ORR_ERR_RANGE
