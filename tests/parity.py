"""Helpers shared by the GPU parity tests: run the HIP path through the C ABI
and compare it with the oracle, element by element."""

from __future__ import annotations

import numpy as np
import torch

import oracle
from barnes_hut_gravitational_amd import orr

# The stated bar for float32 accelerations: max relative per-particle error.
ACC_REL_TOL = 1e-5


def to_dev(pos, mass):
    return torch.from_numpy(np.ascontiguousarray(pos)).cuda(), torch.from_numpy(np.ascontiguousarray(mass)).cuda()


def u32(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint32)


def check_tree(tree: orr.Tree, ot: oracle.Tree):
    """Keys, order, topology and node records bit-exact."""
    info = tree.info()
    assert info["input_status"] == 0
    assert info["n_nodes"] == ot.n_nodes
    assert info["depth"] == ot.depth
    assert info["n_leaves"] == int(ot.is_leaf().sum())
    assert info["max_leaf_count"] == int(ot.count[ot.is_leaf()].max())
    assert np.array_equal(np.array(info["lo"], np.float32).view(np.uint32), ot.lo.view(np.uint32))
    assert np.float32(info["side"]) == ot.side
    ex = tree.export()
    torch.cuda.synchronize()
    assert np.array_equal(ex["keys_sorted"].cpu().numpy().view(np.uint64), ot.keys_sorted)
    assert np.array_equal(u32(ex["perm"]), ot.perm)
    assert np.array_equal(ex["level"].cpu().numpy(), ot.level)
    assert np.array_equal(u32(ex["begin"]), ot.begin)
    assert np.array_equal(u32(ex["count"]), ot.count)
    assert np.array_equal(u32(ex["escape"]), ot.escape)
    assert np.array_equal(u32(ex["s2"]), ot.s2.view(np.uint32))
    assert np.array_equal(u32(ex["geom"]), ot.geom.view(np.uint32))


def rel_err(acc: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """Per-row vector relative error. Both sides must be finite: a NaN or an
    infinity is never within any tolerance (NaN compares false both ways)."""
    assert np.isfinite(acc).all(), "non-finite GPU acceleration"
    assert np.isfinite(ref).all(), "non-finite reference acceleration"
    num = np.linalg.norm(acc.astype(np.float64) - ref, axis=1)
    den = np.linalg.norm(ref.astype(np.float64), axis=1)
    return np.where(den > 0, num / np.where(den > 0, den, 1), np.where(num > 0, np.inf, 0.0))


def check_walk(r: orr.Result, ref: oracle.Result, traversal: str, rows=None):
    """Counts bit-exact, accelerations within ACC_REL_TOL. rows: caller-order
    indices to compare (all if None); ref arrays are indexed like rows."""
    sel = slice(None) if rows is None else rows
    acc = r.acc.cpu().numpy()[sel]
    assert rel_err(acc, ref.acc).max() <= ACC_REL_TOL
    assert np.array_equal(u32(r.visits_own)[sel], ref.visits_own)
    assert np.array_equal(u32(r.n_pp)[sel], ref.n_pp)
    assert np.array_equal(u32(r.n_pc)[sel], ref.n_pc)
    stepped = ref.visits_stepped if traversal == "coherent" else ref.visits_own
    assert np.array_equal(u32(r.visits_stepped)[sel], stepped)


def check_acc_bitwise(r: orr.Result, ref_acc: np.ndarray, rows=None):
    sel = slice(None) if rows is None else rows
    assert np.isfinite(ref_acc).all(), "non-finite reference acceleration"
    assert np.array_equal(r.acc.cpu().numpy()[sel].view(np.uint32), ref_acc.view(np.uint32))


def host_wave_cost(ex, n):
    """The coherent walk's per-wave cost estimate recomputed on the host from an
    exported tree (Tree.export()): for each wave of 64 consecutive sorted
    targets, the summed level of its targets' leaves plus 32 times the levels
    between its deepest leaf and the smallest cell holding all its targets
    (whole 3-bit digits of the common prefix of its first and last key)."""
    keys = ex["keys_sorted"].cpu().numpy().view(np.uint64)
    level = ex["level"].cpu().numpy().astype(np.int64)
    begin, count, escape = (u32(ex[k_]).astype(np.int64) for k_ in ("begin", "count", "escape"))
    leaf = escape == np.arange(len(escape)) + 1
    lvl = np.repeat(level[leaf], count[leaf])  # leaves in preorder cover the sorted targets in order
    assert len(lvl) == n and np.array_equal(begin[leaf], np.concatenate([[0], np.cumsum(count[leaf])[:-1]]))
    nw = (n + 63) // 64
    pad = np.full(64 * nw, -1, np.int64)
    pad[:n] = lvl
    pad = pad.reshape(nw, 64)
    depth_sum = np.where(pad >= 0, pad, 0).sum(axis=1)
    deepest = pad.max(axis=1)
    first_key = keys[0::64].astype(np.uint64)
    last_key = keys[np.minimum(np.arange(nw) * 64 + 63, n - 1)]
    x = first_key ^ last_key
    bl = np.array([int(v).bit_length() for v in x.tolist()], np.int64)
    enclosing = np.where(x == 0, 21, (64 - bl - 1) // 3)
    return depth_sum + 32 * np.maximum(0, deepest - enclosing)
