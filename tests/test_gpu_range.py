"""GPU parity of the range walk (orr_tree_walk_range) and of the split into
cost-balanced ranges (orr_tree_shard_bounds): the share of the targets one
GPU walks when they are split over several. Given the tree, every target's
walk is independent of the others (ADR-0029, Consequences), so walking the
ranges one after another must reproduce the whole walk bit for bit, for both
traversals, and each range must write its own targets' outputs and nothing
else. The oracle checks a range directly, and the bounds are recomputed on
the host from the exported tree: the per-wave cost estimate (summed leaf
level of the wave's targets plus 32 per level between its deepest leaf and
the smallest cell holding all of them) and the split rule."""

import numpy as np
import pytest
import torch

import oracle
from barnes_hut_gravitational_amd import inputs, orr

from parity import host_wave_cost, to_dev, u32

pytestmark = pytest.mark.gpu
EPS, THETA = inputs.EPS, inputs.THETA
SENT_F = np.uint32(0x7FC0DEAD)  # a NaN bit pattern no walk writes
SENT_U = 0x5EEDF00D


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    orr.lib()


def sentinel_outputs(n, device):
    acc = torch.from_numpy(np.full((n, 3), SENT_F, np.uint32).view(np.float32)).to(device)
    cnt = [torch.full((n,), SENT_U, dtype=torch.int32, device=device) for _ in range(4)]
    return acc, cnt


def as_u32(r):
    return [r.acc.cpu().numpy().view(np.uint32)] + [u32(x) for x in
                                                     (r.visits_own, r.visits_stepped, r.n_pp, r.n_pc)]


def expected_bounds(ex, n, cap, k):
    """The split rule of orr_tree_shard_bounds over the cost estimate,
    recomputed from the exported tree."""
    cost = host_wave_cost(ex, n)
    nw = len(cost)
    total = int(cost.sum())
    pre = np.concatenate([[0], np.cumsum(cost)])
    b = [0]
    for j in range(1, k):
        w = int(np.argmax(pre * k >= j * total)) if (pre * k >= j * total).any() else nw
        b.append(min(64 * w, n))
    b.append(n)
    return b


def check_ranges(pos, mass, cap, k, traversal, against_oracle=True):
    n = len(mass)
    P, M = to_dev(pos, mass)
    tree = orr.Tree(P, M, cap)
    print(f"[case] range walk n={n} cap={cap} k={k} {traversal}", flush=True)
    bounds = tree.shard_bounds(k)
    assert len(bounds) == k + 1 and bounds[0] == 0 and bounds[-1] == n
    assert all(a <= b for a, b in zip(bounds, bounds[1:]))
    assert all(b % 64 == 0 for b in bounds[:-1])
    ex = tree.export()
    torch.cuda.synchronize()
    assert bounds == expected_bounds(ex, n, cap, k)
    whole = as_u32(tree.walk(EPS, THETA, traversal=traversal))
    out = sentinel_outputs(n, P.device)
    for a, b in zip(bounds, bounds[1:]):
        tree.walk_range(a, b - a, EPS, THETA, traversal=traversal, out=out)
    torch.cuda.synchronize()
    got = as_u32(orr.Result(out[0], *out[1], None))
    for x, y in zip(got, whole):
        assert np.array_equal(x, y)
    if against_oracle:
        ref = oracle.evaluate(pos, mass, EPS, THETA, cap)
        for x, y in zip(got, (ref.acc.view(np.uint32), ref.visits_own,
                              ref.visits_stepped if traversal == "coherent" else ref.visits_own,
                              ref.n_pp, ref.n_pc)):
            assert np.array_equal(x, y)


@pytest.mark.parametrize("traversal", ["coherent", "independent"])
@pytest.mark.parametrize("kind,n,cap,k", [("plummer", 16384, 32, 8), ("merger", 5000, 16, 3),
                                          ("uniform", 4097, 32, 5), ("plummer", 200, 8, 8),
                                          ("plummer", 1, 32, 2)])
def test_ranges_reproduce_the_walk(kind, n, cap, k, traversal):
    pos, mass = inputs.make(kind, n)
    check_ranges(pos, mass, cap, k, traversal)


@pytest.mark.parametrize("name,k", [("plummer_131k", 8), ("merger_8m", 8), ("merger_8m", 2)])
def test_ranges_configs(name, k):
    """Eight ranges of the 8M merger give each range's schedule lists of at
    most 2,048 waves (longest first); two ranges give lists of about 8,192
    waves, which run their head in list order and their tail longest first."""
    pos, mass = inputs.make_config(name)
    check_ranges(pos, mass, inputs.LEAF_CAP, k, "coherent", against_oracle=False)


def test_range_writes_only_its_targets_and_matches_oracle():
    pos, mass = inputs.make("plummer", 3000)
    n, cap = len(mass), 16
    P, M = to_dev(pos, mass)
    tree = orr.Tree(P, M, cap)
    ot = oracle.build_tree(pos, mass, cap)
    first, count = 640, 1024
    print(f"[case] one range [{first}, {first + count}) of n={n}", flush=True)
    for traversal in ("coherent", "independent"):
        out = sentinel_outputs(n, P.device)
        tree.walk_range(first, count, EPS, THETA, traversal=traversal, out=out)
        torch.cuda.synchronize()
        got = as_u32(orr.Result(out[0], *out[1], None))
        mine = np.zeros(n, bool)
        mine[ot.perm[first:first + count]] = True
        for x in got:
            rows = x[~mine]
            assert np.all(rows == (SENT_F if x.ndim == 2 else np.uint32(SENT_U)))
        tg = np.arange(first, first + count)
        acc_s, pp_s, pc_s, vis_s = oracle.walk(ot, EPS, THETA, targets=tg)
        dst = ot.perm[tg]
        assert np.array_equal(got[0][dst], acc_s.view(np.uint32))
        assert np.array_equal(got[1][dst], vis_s)
        assert np.array_equal(got[3][dst], pp_s)
        assert np.array_equal(got[4][dst], pc_s)
        if traversal == "coherent":
            stepped = np.repeat(oracle.union_visits(ot, EPS, THETA, 64, groups=np.arange(first // 64,
                                                                                      (first + count) // 64)), 64)
            assert np.array_equal(got[2][dst], stepped)
        else:
            assert np.array_equal(got[2][dst], vis_s)


def test_range_argument_errors():
    pos, mass = inputs.make("plummer", 1000)
    P, M = to_dev(pos, mass)
    tree = orr.Tree(P, M, 32)
    L = orr.lib()
    out = sentinel_outputs(1000, P.device)
    for first, count in [(32, 64), (64, 100), (-64, 64), (0, -1), (960, 64), (1024, 0), (0, 1001)]:
        with pytest.raises(orr.OrrError) as e:
            tree.walk_range(first, count, out=out)
        assert e.value.status == orr.ORR_ERR_RANGE
    tree.walk_range(960, 40, out=out)  # the ragged last wave ends at n
    tree.walk_range(1000, 0, out=out)  # empty: nothing enqueued
    with pytest.raises(orr.OrrError) as e:
        tree.walk_range(0, 64, eps=0.0, out=out)
    assert e.value.status == orr.ORR_ERR_RANGE
    for k in (0, 65537):
        with pytest.raises(orr.OrrError) as e:
            tree.shard_bounds(k)
        assert e.value.status == orr.ORR_ERR_RANGE
    assert L.orr_tree_shard_bounds(tree._h, 4, None) == orr.ORR_ERR_INVALID_ARG
    b = tree.shard_bounds(100)  # more ranges than waves: some are empty
    assert b[0] == 0 and b[-1] == 1000 and all(x <= y for x, y in zip(b, b[1:]))
    torch.cuda.synchronize()
