"""Python front end of the CPU oracle (test infrastructure only).

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. It loads ``liborr_oracle.so`` (plain C,
built by ``oracle/build.py``) and composes its steps in the order of the orrery
performance page's "Where one evaluation goes" table: root cube and Morton
keys, sort, gather, build, moments, walk, scatter. Gather and scatter are NumPy
indexing; everything with arithmetic runs in the C library.

Functions whose result has no independent pin say so in their docstring.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# ORR_ORACLE_LIB: another build of the same source (the sanitizer test)
_LIB_PATH = os.environ.get("ORR_ORACLE_LIB") or os.path.join(_HERE, "liborr_oracle.so")
_lib = None

_f32p = np.ctypeslib.ndpointer(np.float32, flags="C_CONTIGUOUS")
_f64p = np.ctypeslib.ndpointer(np.float64, flags="C_CONTIGUOUS")
_u64p = np.ctypeslib.ndpointer(np.uint64, flags="C_CONTIGUOUS")
_u32p = np.ctypeslib.ndpointer(np.uint32, flags="C_CONTIGUOUS")
_u8p = np.ctypeslib.ndpointer(np.uint8, flags="C_CONTIGUOUS")
_i64p = np.ctypeslib.ndpointer(np.int64, flags="C_CONTIGUOUS")
_i64 = ctypes.c_int64
_f32 = ctypes.c_float


class OracleError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"oracle {what} failed with status {status}")
        self.status = status


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _build

            _build.build()
        L = ctypes.CDLL(_LIB_PATH)
        L.oracle_num_threads.restype = ctypes.c_int
        L.oracle_root_cube.argtypes = [_f32p, _f32p, _i64, _f32p, ctypes.POINTER(_f32), ctypes.POINTER(_f32)]
        L.oracle_root_cube.restype = ctypes.c_int
        L.oracle_interleave.argtypes = [ctypes.c_uint32] * 3
        L.oracle_interleave.restype = ctypes.c_uint64
        L.oracle_morton_keys.argtypes = [_f32p, _i64, _f32p, _f32, _u64p]
        L.oracle_morton_keys.restype = None
        L.oracle_sort.argtypes = [_u64p, _i64, _u32p, _u64p]
        L.oracle_sort.restype = ctypes.c_int
        L.oracle_build.argtypes = [_u64p, _i64, ctypes.c_int32, _i64, _u8p, _u32p, _u32p, _u32p]
        L.oracle_build.restype = _i64
        L.oracle_moments.argtypes = [_f32p, _i64, _u8p, _u32p, _u32p, _u32p, _f32, _f32p, _f32p]
        L.oracle_moments.restype = ctypes.c_int
        walk_head = [_f32p, _i64, _f32p, _f32p, _u32p, _u32p, _u32p, _i64, _f32, _f32]
        L.oracle_walk.argtypes = walk_head + [ctypes.c_void_p, _i64, _f32p, _u32p, _u32p, _u32p]
        L.oracle_walk.restype = None
        L.oracle_walk_trace.argtypes = [_f32p, _f32p, _f32p, _u32p, _u32p, _u32p, _i64, _f32, _f32, _i64,
                                        _u64p, _i64]
        L.oracle_walk_trace.restype = _i64
        L.oracle_union_visits.argtypes = walk_head + [_i64, ctypes.c_void_p, _i64, _u32p]
        L.oracle_union_visits.restype = ctypes.c_int
        L.oracle_group_walk.argtypes = walk_head + [_i64, ctypes.c_int, _u32p, _u32p]
        L.oracle_group_walk.restype = ctypes.c_int
        L.oracle_direct_fp64.argtypes = [_f32p, _f32p, _i64, ctypes.c_double, _i64p, _i64, _f64p]
        L.oracle_direct_fp64.restype = None
        L.oracle_direct_fp32.argtypes = [_f32p, _f32p, _i64, _f32, _i64p, _i64, _f32p]
        L.oracle_walk_descend.argtypes = [_f32p, _i64, _f32p, _f32p, _u32p, _u32p, _u32p, _i64, _f32, _f32, _i64,
                                          _f32p, _u32p, _u32p, _u32p, _u32p]
        L.oracle_walk_descend.restype = ctypes.c_int
        L.oracle_direct_fp32.restype = None
        L.oracle_eps_ok.argtypes = [_f32]
        L.oracle_eps_ok.restype = ctypes.c_int
        L.oracle_set_num_threads.argtypes = [ctypes.c_int]
        L.oracle_set_num_threads.restype = None
        _lib = L
    return _lib


def num_threads() -> int:
    return lib().oracle_num_threads()


def set_num_threads(k: int) -> None:
    """Threads of the OpenMP loops over targets (timing only)."""
    lib().oracle_set_num_threads(int(k))


def max_nodes(n: int, leaf_cap: int) -> int:
    """Upper bound on the node count: at most n leaves (non-empty, disjoint) and,
    on each of the 21 split levels, at most n // (leaf_cap + 1) internal nodes."""
    return n + 21 * (n // (leaf_cap + 1)) + 1


def _f32c(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def root_cube(pos, mass):
    pos, mass = _f32c(pos), _f32c(mass)
    lo = np.zeros(3, np.float32)
    side, scale = _f32(), _f32()
    st = lib().oracle_root_cube(pos.reshape(-1), mass, len(mass), lo, ctypes.byref(side), ctypes.byref(scale))
    if st:
        raise OracleError(st, "root_cube")
    return lo, np.float32(side.value), np.float32(scale.value)


def interleave(qx: int, qy: int, qz: int) -> int:
    return int(lib().oracle_interleave(qx, qy, qz))


def morton_keys(pos, lo, scale):
    pos = _f32c(pos)
    keys = np.empty(len(pos), np.uint64)
    lib().oracle_morton_keys(pos.reshape(-1), len(pos), _f32c(lo), _f32(scale), keys)
    return keys


def sort(keys):
    keys = np.ascontiguousarray(keys, dtype=np.uint64)
    perm = np.empty(len(keys), np.uint32)
    ks = np.empty(len(keys), np.uint64)
    st = lib().oracle_sort(keys, len(keys), perm, ks)
    if st:
        raise OracleError(st, "sort")
    return perm, ks


@dataclass
class Tree:
    n: int
    leaf_cap: int
    lo: np.ndarray
    side: np.float32
    scale: np.float32
    keys: np.ndarray          # caller order, uint64
    perm: np.ndarray          # sorted position -> caller index, uint32
    keys_sorted: np.ndarray   # uint64
    xs: np.ndarray            # sorted (x, y, z, m), float32 [n, 4]
    level: np.ndarray         # uint8 [n_nodes]
    begin: np.ndarray         # uint32
    count: np.ndarray         # uint32
    escape: np.ndarray        # uint32
    geom: np.ndarray          # float32 [n_nodes, 4] = (com, M)
    s2: np.ndarray            # float32 [n_nodes]

    @property
    def n_nodes(self) -> int:
        return len(self.level)

    @property
    def depth(self) -> int:
        return int(self.level.max())

    def is_leaf(self):
        return self.escape == np.arange(1, self.n_nodes + 1, dtype=np.uint32)


def build_topology(keys_sorted, leaf_cap):
    n = len(keys_sorted)
    cap_nodes = max_nodes(n, leaf_cap)
    level = np.empty(cap_nodes, np.uint8)
    begin = np.empty(cap_nodes, np.uint32)
    count = np.empty(cap_nodes, np.uint32)
    escape = np.empty(cap_nodes, np.uint32)
    nn = lib().oracle_build(np.ascontiguousarray(keys_sorted, np.uint64), n, leaf_cap, cap_nodes,
                            level, begin, count, escape)
    if nn < 0:
        raise OracleError(-1, "build (node bound exceeded)")
    return level[:nn].copy(), begin[:nn].copy(), count[:nn].copy(), escape[:nn].copy()


def moments(xs, level, begin, count, escape, side):
    nn = len(level)
    geom = np.empty((nn, 4), np.float32)
    s2 = np.empty(nn, np.float32)
    st = lib().oracle_moments(_f32c(xs).reshape(-1), nn, level, begin, count, escape, _f32(side),
                              geom.reshape(-1), s2)
    if st:
        raise OracleError(st, "moments")
    return geom, s2


def build_tree(pos, mass, leaf_cap=32) -> Tree:
    pos, mass = _f32c(pos), _f32c(mass)
    lo, side, scale = root_cube(pos, mass)
    keys = morton_keys(pos, lo, scale)
    perm, ks = sort(keys)
    xs = np.empty((len(mass), 4), np.float32)
    xs[:, :3] = pos[perm]
    xs[:, 3] = mass[perm]
    level, begin, count, escape = build_topology(ks, leaf_cap)
    geom, s2 = moments(xs, level, begin, count, escape, side)
    return Tree(len(mass), leaf_cap, lo, side, scale, keys, perm, ks, xs, level, begin, count, escape, geom, s2)


def check_eps(eps):
    """Raise unless the target's own term m * 0 * eps^-3 is +0, i.e. eps^-3 as
    the term evaluates it in float32 is finite (about eps >= 1.43e-13)."""
    if not lib().oracle_eps_ok(_f32(eps)):
        raise OracleError(2, f"eps = {eps!r} (own term 0 * eps^-3 is not +0)")


def _walk_args(t: Tree, eps, theta):
    check_eps(eps)
    return (t.xs.reshape(-1), t.n, t.geom.reshape(-1), t.s2, t.begin, t.count, t.escape, t.n_nodes,
            _f32(eps), _f32(theta))


def walk(t: Tree, eps, theta, targets=None):
    """Stackless walk for sorted targets (all if None). Returns sorted-order
    (acc [m,3] f32, pp, pc, visits) indexed like `targets`."""
    if targets is None:
        m, tp = t.n, None
    else:
        targets = np.ascontiguousarray(targets, np.int64)
        m, tp = len(targets), targets.ctypes.data_as(ctypes.c_void_p)
    acc = np.empty((m, 3), np.float32)
    pp = np.empty(m, np.uint32)
    pc = np.empty(m, np.uint32)
    vis = np.empty(m, np.uint32)
    lib().oracle_walk(*_walk_args(t, eps, theta), tp, m, acc.reshape(-1), pp, pc, vis)
    return acc, pp, pc, vis


def walk_descend(t: Tree, eps, theta, width):
    """The descend-together group walk (ADR-0029, Alternatives considered):
    groups of `width` consecutive sorted targets open a node when any member
    would. Returns sorted-order (acc [n,3] f32, pp, pc, visits, covered)."""
    check_eps(eps)
    n = t.n
    acc = np.empty((n, 3), np.float32)
    pp, pc, vis, cov = (np.empty(n, np.uint32) for _ in range(4))
    st = lib().oracle_walk_descend(t.xs.reshape(-1), n, t.geom.reshape(-1), t.s2, t.begin, t.count, t.escape,
                                   t.n_nodes, _f32(eps), _f32(theta), int(width), acc.reshape(-1), pp, pc, vis,
                                   cov)
    if st != 0:
        raise OracleError(st, "walk_descend")
    return acc, pp, pc, vis, cov


def walk_trace(t: Tree, eps, theta, target):
    """Visit sequence of one sorted target: (node [k], action [k]) with action
    0 = accepted, 1 = opened leaf, 2 = opened internal node."""
    check_eps(eps)
    buf = np.empty(t.n_nodes, np.uint64)
    k = lib().oracle_walk_trace(t.xs.reshape(-1), t.geom.reshape(-1), t.s2, t.begin, t.count, t.escape,
                                t.n_nodes, _f32(eps), _f32(theta), int(target), buf, len(buf))
    return (buf[:k] >> np.uint64(2)).astype(np.int64), (buf[:k] & np.uint64(3)).astype(np.int64)


def union_visits(t: Tree, eps, theta, width=64, groups=None):
    """Per group of `width` consecutive sorted targets (all groups, or the
    listed group indices): size of the union of the members' visited node sets."""
    if groups is None:
        m, gp = (t.n + width - 1) // width, None
    else:
        groups = np.ascontiguousarray(groups, np.int64)
        m, gp = len(groups), groups.ctypes.data_as(ctypes.c_void_p)
    out = np.empty(m, np.uint32)
    st = lib().oracle_union_visits(*_walk_args(t, eps, theta), width, gp, m, out)
    if st:
        raise OracleError(st, "union_visits")
    return out


def group_walk(t: Tree, eps, theta, width=64, rule="min"):
    """Simulated group walk. rule 'min' moves to the minimum wanted index;
    'ballot' moves to node+1 if any acting lane descends, else to the escape.
    Returns (steps per group, own visits per sorted target, ok)."""
    groups = (t.n + width - 1) // width
    steps = np.empty(groups, np.uint32)
    own = np.empty(t.n, np.uint32)
    bad = lib().oracle_group_walk(*_walk_args(t, eps, theta), width, 0 if rule == "min" else 1, steps, own)
    return steps, own, bad == 0


def direct_fp32(pos, mass, eps, targets=None):
    """Float32 direct sum in index order with the walk's term, for caller-order
    targets (all if None); the target's own term (+0) is included."""
    check_eps(eps)
    pos, mass = _f32c(pos), _f32c(mass)
    n = len(mass)
    targets = np.arange(n, dtype=np.int64) if targets is None else np.ascontiguousarray(targets, np.int64)
    acc = np.empty((len(targets), 3), np.float32)
    lib().oracle_direct_fp32(pos.reshape(-1), mass, n, _f32(eps), targets, len(targets), acc.reshape(-1))
    return acc


def direct_fp64(pos, mass, eps, targets=None):
    """Compensated float64 direct sum for caller-order targets (all if None)."""
    pos, mass = _f32c(pos), _f32c(mass)
    n = len(mass)
    targets = np.arange(n, dtype=np.int64) if targets is None else np.ascontiguousarray(targets, np.int64)
    acc = np.empty((len(targets), 3), np.float64)
    lib().oracle_direct_fp64(pos.reshape(-1), mass, n, float(eps), targets, len(targets), acc.reshape(-1))
    return acc


@dataclass
class Result:
    acc: np.ndarray             # caller order [n, 3] float32
    visits_own: np.ndarray      # uint32, caller order
    visits_stepped: np.ndarray  # uint32, caller order (group union, width 64)
    n_pp: np.ndarray
    n_pc: np.ndarray
    tree: Tree


def evaluate(pos, mass, eps=0.05, theta=0.5, leaf_cap=32, width=64) -> Result:
    """The whole force evaluation: build, walk every target, scatter to caller order."""
    check_eps(eps)
    t = build_tree(pos, mass, leaf_cap)
    acc_s, pp_s, pc_s, vis_s = walk(t, eps, theta)
    groups = union_visits(t, eps, theta, width)
    stepped_s = np.repeat(groups, width)[: t.n]
    n = t.n
    acc = np.empty((n, 3), np.float32)
    acc[t.perm] = acc_s
    out = []
    for a in (vis_s, stepped_s, pp_s, pc_s):
        b = np.empty(n, np.uint32)
        b[t.perm] = a
        out.append(b)
    return Result(acc, out[0], out[1], out[2], out[3], t)
