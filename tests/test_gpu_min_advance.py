"""GPU parity of the coherent walk that advances by an explicit wave minimum
of the lanes' next nodes (orr_tree_walk_min_advance; the sub-group advance of
the orrery solver page, "The mitigation"). The minimum of the lanes' next
nodes is c + 1 when some lane opened c and the escape of c otherwise, so
this walk visits the same nodes in the same order as the coherent walk's
mask select: every output must equal the oracle's bit for bit, and
visits_stepped the coherent walk's (the oracle's union of each wave's walks)."""

import numpy as np
import pytest
import torch

import oracle
from barnes_hut_gravitational_amd import inputs, orr

from parity import to_dev, u32

pytestmark = pytest.mark.gpu
EPS, THETA = inputs.EPS, inputs.THETA


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    orr.lib()


def check_min_advance(pos, mass, cap, theta=THETA, against_oracle=True):
    P, M = to_dev(pos, mass)
    tree = orr.Tree(P, M, cap)
    print(f"[case] min-advance n={len(mass)} cap={cap} theta={theta}", flush=True)
    a = tree.walk(EPS, theta, traversal="coherent")
    b = tree.walk_min_advance(EPS, theta)
    torch.cuda.synchronize()
    assert torch.equal(a.acc.view(torch.int32), b.acc.view(torch.int32))
    for x, y in ((a.visits_own, b.visits_own), (a.visits_stepped, b.visits_stepped), (a.n_pp, b.n_pp),
                 (a.n_pc, b.n_pc)):
        assert torch.equal(x, y)
    if against_oracle:
        ref = oracle.evaluate(pos, mass, EPS, theta, cap)
        assert np.array_equal(b.acc.cpu().numpy().view(np.uint32), ref.acc.view(np.uint32))
        assert np.array_equal(u32(b.visits_own), ref.visits_own)
        assert np.array_equal(u32(b.visits_stepped), ref.visits_stepped)
        assert np.array_equal(u32(b.n_pp), ref.n_pp)
        assert np.array_equal(u32(b.n_pc), ref.n_pc)


@pytest.mark.parametrize("kind,n,cap", [("plummer", 3000, 16), ("merger", 2000, 32), ("uniform", 4097, 32),
                                        ("plummer", 33, 8), ("plummer", 1, 32), ("plummer", 16384, 32)])
def test_min_advance_small(kind, n, cap):
    pos, mass = inputs.make(kind, n)
    check_min_advance(pos, mass, cap)


@pytest.mark.parametrize("theta", [0.0, 0.3, 1.0, 1e6])
def test_min_advance_thetas(theta):
    pos, mass = inputs.make("plummer", 2500)
    check_min_advance(pos, mass, 16, theta=theta)


def test_min_advance_coincident_points():
    # every particle at one point: a chain of nodes down to level 21
    pos = np.zeros((200, 3), np.float32)
    mass = np.full(200, 1.0 / 200, np.float32)
    check_min_advance(pos, mass, 8)


@pytest.mark.parametrize("name", ["plummer_131k", "uniform_262k"])
def test_min_advance_configs(name):
    pos, mass = inputs.make_config(name)
    check_min_advance(pos, mass, inputs.LEAF_CAP, against_oracle=False)


def test_min_advance_plummer_1m_equals_coherent():
    pos, mass = inputs.make_config("plummer_1m")
    check_min_advance(pos, mass, inputs.LEAF_CAP, against_oracle=False)
