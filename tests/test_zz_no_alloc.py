"""The allocation-free entry point (orr_eval_forces_noalloc) against the
evaluation with a caller workspace (orr_eval_forces), through the C ABI:
every output bit for bit, on consecutive calls that share the library's one
per-GPU workspace array (a second, smaller call sees the first call's
contents), at the largest size the array holds, and against the oracle on a
small case. Sizes beyond the array are refused before any device work."""

import ctypes

import numpy as np
import pytest
import torch

import oracle
from barnes_hut_gravitational_amd import inputs, orr

from parity import check_acc_bitwise, check_walk, to_dev

pytestmark = pytest.mark.gpu
EPS, THETA, CAP = inputs.EPS, inputs.THETA, inputs.LEAF_CAP


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    orr.lib()


def both(pos, mass, cap=CAP, theta=THETA, traversal="coherent"):
    P, M = to_dev(pos, mass)
    a = orr.orr_eval_forces_noalloc(P, M, eps=EPS, theta=theta, leaf_cap=cap, traversal=traversal)
    b = orr.orr_eval_forces(P, M, eps=EPS, theta=theta, leaf_cap=cap, traversal=traversal)
    torch.cuda.synchronize()
    for f in ("acc", "visits_own", "visits_stepped", "n_pp", "n_pc"):
        x, y = getattr(a, f), getattr(b, f)
        assert torch.equal(x.view(torch.int32), y.view(torch.int32)), f
    assert torch.isfinite(a.acc).all()
    return a


def test_consecutive_calls_second_smaller():
    cases = [("plummer", 20001, CAP, THETA, "coherent"), ("uniform", 3000, 8, 0.7, "coherent"),
             ("merger", 777, 32, 0.5, "independent")]
    for kind, n, cap, theta, tr in cases:
        print(f"[case] noalloc {kind} n={n} cap={cap} theta={theta} {tr}", flush=True)
        pos, mass = inputs.make(kind, n)
        r = both(pos, mass, cap, theta, tr)
        ref = oracle.evaluate(pos, mass, EPS, theta, cap)
        check_walk(r, ref, tr)
        check_acc_bitwise(r, ref.acc)


def test_largest_size_the_array_holds():
    n = 1 << 20
    assert orr.workspace_bytes(n, CAP) <= orr.NOALLOC_SCRATCH_BYTES
    print(f"[case] noalloc plummer n={n}", flush=True)
    pos, mass = inputs.make("plummer", n)
    both(pos, mass)
    print("[case] noalloc plummer n=4096 after the largest", flush=True)
    pos, mass = inputs.make("plummer", 4096)
    both(pos, mass)


def test_sizes_beyond_the_array_are_refused():
    L = orr.lib()
    for n, cap in ((1100000, 32), (1 << 20, 1), (1 << 30, 32)):
        assert orr.workspace_bytes(n, cap) > orr.NOALLOC_SCRATCH_BYTES
        st = L.orr_eval_forces_noalloc(1, 1, n, EPS, THETA, cap, 1, None, None, None, None, None, None)
        assert st == orr.ORR_ERR_WORKSPACE, (n, cap)
        assert b"allocation-free" in L.orr_last_error()
    assert L.orr_eval_forces_noalloc(None, 1, 100, EPS, THETA, CAP, 1, None, None, None, None, None,
                                     None) == orr.ORR_ERR_INVALID_ARG
    assert L.orr_eval_forces_noalloc(1, 1, 100, 0.0, THETA, CAP, 1, None, None, None, None, None,
                                     None) == orr.ORR_ERR_RANGE
