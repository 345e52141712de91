"""The coherent walk's schedule (orr_tree_export_schedule), recomputed on the
host from the exported tree. The schedule decides only when each wave of 64
consecutive sorted targets runs (the orrery solver page, "The mitigation"),
never what it computes. The parity tests show that every target is walked.
This file pins the rest:
- the per-wave cost estimate;
- the eight per-XCD lists (64 contiguous regions, dealt as Morton eighths or
  in a snake over their cost);
- each list's order: longest first for a list of at most two tails, else its
  head in list order and its tail of the cheapest waves, longest first."""

import numpy as np
import pytest
import torch

from barnes_hut_gravitational_amd import inputs, orr

from parity import host_wave_cost, to_dev, u32

pytestmark = pytest.mark.gpu
KBINS, TAIL, REGIONS, SLACK = 2048, 1024, 64, 5


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    orr.lib()


def expected_lists(cost):
    """The waves of each XCD list in list order, from the clamped costs."""
    nw = len(cost)
    R = -(-nw // REGIONS)
    rc = np.array([int(cost[r * R:min(r * R + R, nw)].sum()) for r in range(REGIONS)], np.int64)
    eighths = rc.reshape(8, REGIONS // 8).sum(axis=1)
    if eighths.max() * 800 <= eighths.sum() * (100 + SLACK):
        owner = np.arange(REGIONS) // (REGIONS // 8)
    else:
        owner = np.empty(REGIONS, np.int64)
        for r in range(REGIONS):
            rank = int(np.sum((rc > rc[r]) | ((rc == rc[r]) & (np.arange(REGIONS) < r))))
            owner[r] = 7 - rank % 8 if (rank // 8) % 2 else rank % 8
    lists = []
    for x in range(8):
        lists.append([w for r in range(REGIONS) if owner[r] == x for w in range(r * R, min(r * R + R, nw))])
    return lists, 8 * R


def check_schedule(kind, n):
    pos, mass = inputs.make(kind, n)
    print(f"[case] schedule {kind} n={n}", flush=True)
    P, M = to_dev(pos, mass)
    tree = orr.Tree(P, M, inputs.LEAF_CAP)
    sch = tree.export_schedule()
    ex = tree.export()
    torch.cuda.synchronize()
    cost = u32(sch["wave_cost"]).astype(np.int64)
    assert np.array_equal(cost, host_wave_cost(ex, n))
    c = np.minimum(cost, KBINS - 1)
    order = u32(sch["order"]).astype(np.int64)
    lists, L = expected_lists(c)
    hybrid = 0
    for x, waves in enumerate(lists):
        ln = len(waves)
        assert order[8 * L + x] == ln, x
        got = order[x * L:x * L + ln]
        head = []
        if ln > 2 * TAIL:
            hybrid += 1
            cut = np.sort(c[waves])[::-1][ln - TAIL]  # cost at decreasing-cost position len - TAIL
            head = [w for w in waves if c[w] > cut]
        assert got[:len(head)].tolist() == head, x
        tail = got[len(head):]
        assert sorted(tail.tolist()) == sorted(set(waves) - set(head)), x
        assert np.all(np.diff(c[tail]) <= 0), x
        assert len(head) == 0 or len(tail) >= TAIL
    return hybrid


@pytest.mark.parametrize("kind,n", [("plummer", 1000), ("plummer", 16384), ("uniform", 262144),
                                     ("plummer", 1048576)])
def test_schedule_longest_first(kind, n):
    """Lists of at most two tails (here every list) run longest first."""
    assert check_schedule(kind, n) == 0


@pytest.mark.parametrize("kind,n", [("plummer", 3000017), ("merger", 8388608)])
def test_schedule_head_and_tail(kind, n):
    """Long lists: the head keeps list order, the tail runs longest first.
    3,000,017 targets leave a ragged last wave and a short last region."""
    assert check_schedule(kind, n) == 8
