"""Pins of the oracle's descend-together group walk, the alternative ADR-0029
rejects ("Alternatives considered"): a group of targets opens a node when any
member would, the members that would have accepted it descending too.

Pins: a group of one is the masked walk itself (bit for bit); at theta = 0 it
is the sorted direct sum; every target's terms account for every particle
exactly once; the result depends on the group (it differs between widths);
and it is at least as accurate as the masked walk against the
double-precision direct sum while doing more particle terms, which is the
trade the ADR describes.
"""

import numpy as np
import pytest

import oracle
from barnes_hut_gravitational_amd import inputs

from test_oracle_walk import fp32_direct_sorted

EPS, THETA = 0.05, 0.5


def bits(a):
    return np.ascontiguousarray(a, np.float32).view(np.uint32)


@pytest.mark.parametrize("kind,n,cap", [("plummer", 3000, 16), ("merger", 2500, 32), ("uniform", 2000, 8)])
def test_width_one_is_the_masked_walk(kind, n, cap):
    pos, mass = inputs.make(kind, n)
    t = oracle.build_tree(pos, mass, cap)
    acc, pp, pc, vis, cov = oracle.walk_descend(t, EPS, THETA, 1)
    racc, rpp, rpc, rvis = oracle.walk(t, EPS, THETA)
    assert np.array_equal(bits(acc), bits(racc))
    assert np.array_equal(pp, rpp) and np.array_equal(pc, rpc) and np.array_equal(vis, rvis)


def test_theta_zero_is_the_sorted_direct_sum():
    pos, mass = inputs.make("plummer", 400)
    t = oracle.build_tree(pos, mass, 8)
    acc, pp, pc, vis, cov = oracle.walk_descend(t, EPS, 0.0, 64)
    assert np.array_equal(bits(acc), bits(fp32_direct_sorted(t.xs, EPS)))
    assert np.all(pc == 0) and np.all(pp == t.n - 1) and np.all(vis == t.n_nodes)


@pytest.mark.parametrize("width", [2, 7, 32, 64])
@pytest.mark.parametrize("kind", ["plummer", "merger"])
def test_every_particle_summed_once(kind, width):
    pos, mass = inputs.make(kind, 3001)
    t = oracle.build_tree(pos, mass, 16)
    acc, pp, pc, vis, cov = oracle.walk_descend(t, EPS, THETA, width)
    assert np.all(cov == t.n)
    # the group's steps are the same for every member of a group
    g = np.arange(t.n) // width
    for k in np.unique(g)[:50]:
        assert len(set(vis[g == k].tolist())) == 1


def test_result_depends_on_the_group():
    pos, mass = inputs.make("plummer", 4096)
    t = oracle.build_tree(pos, mass, 32)
    a16 = oracle.walk_descend(t, EPS, THETA, 16)[0]
    a64 = oracle.walk_descend(t, EPS, THETA, 64)[0]
    assert not np.array_equal(bits(a16), bits(a64))


def test_more_accurate_and_more_work_than_masking():
    pos, mass = inputs.make("plummer", 16384)
    t = oracle.build_tree(pos, mass, 32)
    acc_d, pp_d, pc_d, vis_d, _ = oracle.walk_descend(t, EPS, THETA, 64)
    acc_m, pp_m, pc_m, vis_m = oracle.walk(t, EPS, THETA)
    rows = np.arange(0, t.n, 7)
    ref = oracle.direct_fp64(t.xs[:, :3], t.xs[:, 3], EPS, rows)
    def rms(a):
        e = np.linalg.norm(a[rows] - ref, axis=1) / np.linalg.norm(ref, axis=1)
        return np.sqrt(np.mean(e ** 2))
    assert rms(acc_d) < rms(acc_m)
    assert pp_d.sum() > pp_m.sum() and (pp_d.astype(np.int64) + pc_d).sum() > (pp_m.astype(np.int64) + pc_m).sum()
    assert np.all(pp_d >= pp_m)
