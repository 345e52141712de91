"""CPU-side checks of the C ABI: the built library loads, exports every entry
point include/orr.h declares, and rejects bad arguments before any device
work (no GPU is touched by these calls)."""

import ctypes
import os
import re
import subprocess

import pytest

from barnes_hut_gravitational_amd import orr

from eps_bound import self_term_finite, smallest_eps

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "orr.h")


def declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(orr_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_binding_names():
    assert declared() == sorted(orr.EXPORTED)


def test_library_exports_every_declared_symbol():
    L = orr.lib()
    for name in declared():
        assert hasattr(L, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", orr.LIB_PATH], capture_output=True, text=True).stdout
    syms = set(l.split()[-1] for l in out.splitlines() if l.strip())
    assert set(declared()) <= syms


def test_checked_build_exports_the_same_symbols():
    """The checked build (device index checks) is the same ABI: every
    declared entry point, loaded without a GPU call."""
    from barnes_hut_gravitational_amd import build_lib

    assert os.path.exists(build_lib.CHECKED_LIB), "run __graft_entry__.build()"
    out = subprocess.run(["nm", "-D", "--defined-only", build_lib.CHECKED_LIB], capture_output=True, text=True).stdout
    syms = set(l.split()[-1] for l in out.splitlines() if l.strip())
    assert set(declared()) <= syms
    L = ctypes.CDLL(build_lib.CHECKED_LIB)
    L.orr_abi_version.restype = ctypes.c_int
    assert L.orr_abi_version() == orr.abi_version()


def test_static_strings_and_version():
    L = orr.lib()
    assert orr.abi_version() == 2
    assert L.orr_traversal_name(0) == b"independent" and L.orr_traversal_name(1) == b"coherent"
    assert L.orr_traversal_name(7) == b"invalid"
    assert L.orr_status_string(0) == b"ok" and L.orr_status_string(5) == b"workspace too small"
    assert L.orr_status_string(99) == b"unknown status"


def test_workspace_bytes():
    assert orr.workspace_bytes(0, 32) == 0
    assert orr.workspace_bytes(100, 0) == 0 and orr.workspace_bytes(100, 257) == 0
    assert orr.workspace_bytes(2**31, 32) == 0
    assert orr.workspace_bytes(2**31 - 1, 32) > 0
    a, b = orr.workspace_bytes(1 << 20, 32), orr.workspace_bytes(1 << 20, 1)
    assert 0 < a < b
    assert a % 256 == 0
    # grows with n
    assert orr.workspace_bytes(1000, 32) < orr.workspace_bytes(2000, 32)


def node_bound(n, cap):
    return n + 21 * (n // (cap + 1)) + 1


@pytest.mark.parametrize("cap", [1, 2, 8, 19])
def test_node_bound_limited_to_32_bit_indices(cap):
    """Node indices are 32-bit on the device: the largest n whose node bound
    n + 21 floor(n / (cap + 1)) + 1 is at most 2^32 - 1 is accepted and the
    next one refused, by the size query and by the entry points, before any
    device work. From leaf capacity 20 on, every n up to ORR_MAX_N fits."""
    lo, hi = 1, 2**31 - 1
    while lo < hi:  # the largest n whose bound fits
        m = (lo + hi + 1) // 2
        lo, hi = (m, hi) if node_bound(m, cap) <= 2**32 - 1 else (lo, m - 1)
    assert node_bound(lo, cap) <= 2**32 - 1 < node_bound(lo + 1, cap)
    assert orr.workspace_bytes(lo, cap) > 0
    assert orr.workspace_bytes(lo + 1, cap) == 0
    st, msg = _eval(n=lo + 1, cap=cap)
    assert st == orr.ORR_ERR_RANGE and "32-bit node indices" in msg
    h = ctypes.c_void_p()
    assert orr.lib().orr_build_tree(1, 1, lo + 1, cap, 256, 1 << 30, None, ctypes.byref(h)) == orr.ORR_ERR_RANGE
    assert h.value is None
    if cap == 1:
        assert lo == 373_475_417


def test_no_node_bound_limit_from_leaf_capacity_20():
    assert node_bound(2**31 - 1, 20) <= 2**32 - 1
    assert orr.workspace_bytes(2**31 - 1, 20) > 0


def _eval(**kw):
    L = orr.lib()
    args = dict(pos=1, mass=1, n=100, eps=0.05, theta=0.5, cap=32, tr=1, ws=256, ws_bytes=1 << 30)
    args.update(kw)
    st = L.orr_eval_forces(args["pos"], args["mass"], args["n"], args["eps"], args["theta"], args["cap"],
                           args["tr"], None, None, None, None, None, args["ws"], args["ws_bytes"], None, None)
    return st, L.orr_last_error().decode()


@pytest.mark.parametrize("kw,status", [
    ({"n": 0}, orr.ORR_ERR_RANGE), ({"n": -5}, orr.ORR_ERR_RANGE), ({"n": 2**31}, orr.ORR_ERR_RANGE),
    ({"cap": 0}, orr.ORR_ERR_RANGE), ({"cap": 300}, orr.ORR_ERR_RANGE),
    ({"eps": 0.0}, orr.ORR_ERR_RANGE), ({"eps": -1.0}, orr.ORR_ERR_RANGE), ({"eps": float("inf")}, orr.ORR_ERR_RANGE),
    ({"eps": float("nan")}, orr.ORR_ERR_RANGE), ({"theta": -0.1}, orr.ORR_ERR_RANGE),
    ({"theta": float("nan")}, orr.ORR_ERR_RANGE), ({"tr": 2}, orr.ORR_ERR_INVALID_ARG),
    ({"pos": None}, orr.ORR_ERR_INVALID_ARG), ({"mass": None}, orr.ORR_ERR_INVALID_ARG),
    ({"ws": None}, orr.ORR_ERR_INVALID_ARG), ({"ws": 256 + 8}, orr.ORR_ERR_INVALID_ARG),
    ({"ws_bytes": 1000}, orr.ORR_ERR_WORKSPACE)])
def test_eval_argument_errors(kw, status):
    st, msg = _eval(**kw)
    assert st == status and msg


def test_build_and_walk_argument_errors():
    L = orr.lib()
    h = ctypes.c_void_p()
    assert L.orr_build_tree(1, 1, 100, 32, 256, 1 << 30, None, None) == orr.ORR_ERR_INVALID_ARG
    assert L.orr_build_tree(1, 1, 0, 32, 256, 1 << 30, None, ctypes.byref(h)) == orr.ORR_ERR_RANGE
    assert h.value is None
    assert L.orr_tree_walk(None, 0.05, 0.5, 1, None, None, None, None, None, None) == orr.ORR_ERR_INVALID_ARG
    assert L.orr_tree_walk_grouped(None, 0.05, 0.5, 32, None, None, None, None, None) == orr.ORR_ERR_INVALID_ARG
    assert L.orr_tree_walk_descend(None, 0.05, 0.5, 32, None, None, None, None, None) == orr.ORR_ERR_INVALID_ARG
    assert L.orr_tree_walk_min_advance(None, 0.05, 0.5, None, None, None, None, None) == orr.ORR_ERR_INVALID_ARG
    assert L.orr_tree_walk_width(None, 0.05, 0.5, 64, None, None, None, None, None) == orr.ORR_ERR_INVALID_ARG
    assert L.orr_tree_walk_range(None, 0.05, 0.5, 1, 0, 64, None, None, None, None, None) == orr.ORR_ERR_INVALID_ARG
    assert L.orr_tree_shard_bounds(None, 8, None) == orr.ORR_ERR_INVALID_ARG
    assert L.orr_tree_info_get(None, None) == orr.ORR_ERR_INVALID_ARG
    assert L.orr_tree_check(None) == orr.ORR_ERR_INVALID_ARG
    assert L.orr_workspace_check(None, 1 << 20, None) == orr.ORR_ERR_INVALID_ARG
    assert L.orr_workspace_check(256 + 8, 1 << 20, None) == orr.ORR_ERR_INVALID_ARG
    assert L.orr_workspace_check(256, 64, None) == orr.ORR_ERR_WORKSPACE
    assert L.orr_tree_export(None, None, None, None, None, None, None, None, None) == orr.ORR_ERR_INVALID_ARG
    assert L.orr_selftest_inv_sqrt(0, 1, None, 1, None) == orr.ORR_ERR_INVALID_ARG
    assert L.orr_selftest_inv_sqrt(5, 1, 1, 1, None) == orr.ORR_ERR_INVALID_ARG
    L.orr_tree_free(None)


@pytest.mark.parametrize("args,status", [
    ((None, 1, 100, 0.05, 1), orr.ORR_ERR_INVALID_ARG), ((1, None, 100, 0.05, 1), orr.ORR_ERR_INVALID_ARG),
    ((1, 1, 100, 0.05, None), orr.ORR_ERR_INVALID_ARG), ((1, 1, 0, 0.05, 1), orr.ORR_ERR_RANGE),
    ((1, 1, 2**31, 0.05, 1), orr.ORR_ERR_RANGE), ((1, 1, 100, 0.0, 1), orr.ORR_ERR_RANGE),
    ((1, 1, 100, float("nan"), 1), orr.ORR_ERR_RANGE), ((1, 1, 100, float("inf"), 1), orr.ORR_ERR_RANGE)])
def test_direct_argument_errors(args, status):
    L = orr.lib()
    pos, mass, n, eps, acc = args
    assert L.orr_direct_forces(pos, mass, n, eps, acc, None) == status
    assert L.orr_last_error().decode()


def test_binding_rejects_host_tensors():
    import torch

    with pytest.raises(orr.OrrError):
        orr.orr_eval_forces(torch.zeros(4, 3), torch.ones(4))


def test_eps_lower_bound():
    """eps is rejected exactly where the own term's eps^-3 overflows float32
    (it would be 0 * inf = NaN on every target). An admitted eps passes on to
    the traversal check (bad traversal 2), so no device work is started."""
    lo, below = smallest_eps()
    assert 1.4e-13 < lo < 1.5e-13 and self_term_finite(lo) and not self_term_finite(below)
    for eps in (1e-30, 1e-20, 1e-14, below):
        assert _eval(eps=eps, tr=2)[0] == orr.ORR_ERR_RANGE, eps
        assert orr.lib().orr_direct_forces(1, 1, 100, eps, 1, None) == orr.ORR_ERR_RANGE
    for eps in (lo, 1e-12, 1e-3, 0.05):
        assert _eval(eps=eps, tr=2)[0] == orr.ORR_ERR_INVALID_ARG, eps


def test_noalloc_limit_and_argument_errors():
    """The allocation-free entry refuses, before any device work, sizes whose
    workspace exceeds its fixed array, and bad arguments as orr_eval_forces."""
    text = open(HEADER).read()
    m = re.search(r"#define ORR_NOALLOC_SCRATCH_BYTES \((\d+)ull << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == orr.NOALLOC_SCRATCH_BYTES
    assert orr.workspace_bytes(1 << 20, 32) <= orr.NOALLOC_SCRATCH_BYTES < orr.workspace_bytes(1100000, 32)
    L = orr.lib()
    for n, cap, status in ((1100000, 32, orr.ORR_ERR_WORKSPACE), ((1 << 20), 1, orr.ORR_ERR_WORKSPACE),
                           (0, 32, orr.ORR_ERR_RANGE), (100, 0, orr.ORR_ERR_RANGE)):
        assert L.orr_eval_forces_noalloc(1, 1, n, 0.05, 0.5, cap, 1, None, None, None, None, None, None) == status
    assert L.orr_eval_forces_noalloc(None, 1, 100, 0.05, 0.5, 32, 1, None, None, None, None, None,
                                     None) == orr.ORR_ERR_INVALID_ARG
    assert L.orr_eval_forces_noalloc(1, 1, 100, 1e-20, 0.5, 32, 1, None, None, None, None, None,
                                     None) == orr.ORR_ERR_RANGE
    assert L.orr_eval_forces_noalloc(1, 1, 100, 0.05, 0.5, 32, 2, None, None, None, None, None,
                                     None) == orr.ORR_ERR_INVALID_ARG


@pytest.mark.parametrize("args,status", [
    ((None, 1, 100, 0.05, 1, 10, 1), orr.ORR_ERR_INVALID_ARG), ((1, 1, 100, 0.05, None, 10, 1), orr.ORR_ERR_INVALID_ARG),
    ((1, 1, 100, 0.05, 1, 10, None), orr.ORR_ERR_INVALID_ARG), ((1, 1, 0, 0.05, 1, 10, 1), orr.ORR_ERR_RANGE),
    ((1, 1, 100, 0.05, 1, -1, 1), orr.ORR_ERR_RANGE), ((1, 1, 100, 1e-20, 1, 10, 1), orr.ORR_ERR_RANGE),
    ((1, 1, 100, 0.05, 1, 0, 1), orr.ORR_OK)])
def test_direct_targets_argument_errors(args, status):
    """Checked before any device work; zero targets is a no-op."""
    L = orr.lib()
    pos, mass, n, eps, targets, m, acc = args
    assert L.orr_direct_forces_targets(pos, mass, n, eps, targets, m, acc, None) == status


@pytest.mark.parametrize("args,status", [
    ((None, 1, 100, 0.05, 1, 10, 1), orr.ORR_ERR_INVALID_ARG), ((1, 1, 100, 0.05, None, 10, 1), orr.ORR_ERR_INVALID_ARG),
    ((1, 1, 0, 0.05, 1, 10, 1), orr.ORR_ERR_RANGE), ((1, 1, 100, -1.0, 1, 10, 1), orr.ORR_ERR_RANGE),
    ((1, 1, 100, float("nan"), 1, 10, 1), orr.ORR_ERR_RANGE), ((1, 1, 100, 0.05, 1, -2, 1), orr.ORR_ERR_RANGE),
    ((1, 1, 100, 0.0, 1, 0, 1), orr.ORR_OK)])
def test_direct_fp64_targets_argument_errors(args, status):
    L = orr.lib()
    pos, mass, n, eps, targets, m, acc = args
    assert L.orr_direct_forces_fp64_targets(pos, mass, n, eps, targets, m, acc, None) == status
