"""ctypes binding of liborr.so (include/orr.h), with the same entry-point names.

Marshalling only: every step of the evaluation runs in the HIP library.
PyTorch supplies device memory (tensors) and the current HIP stream. There is
no fallback: without the built library every call raises.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch  # loaded before liborr so both share one HIP runtime

_HERE = os.path.dirname(os.path.abspath(__file__))
# ORR_CHECKED=1 loads the checked build (the same ABI, with every index a
# kernel takes from device data tested; a failed test makes the next
# synchronising call return ORR_ERR_HIP).
LIB_PATH = os.path.join(_HERE, "liborr_checked.so" if os.environ.get("ORR_CHECKED") == "1" else "liborr.so")

(ORR_OK, ORR_ERR_INVALID_ARG, ORR_ERR_RANGE, ORR_ERR_NONFINITE, ORR_ERR_HIP, ORR_ERR_WORKSPACE,
 ORR_ERR_HOST_MEMORY) = range(7)
TRAVERSALS = {"independent": 0, "coherent": 1}
NOALLOC_SCRATCH_BYTES = 144 << 20  # ORR_NOALLOC_SCRATCH_BYTES of include/orr.h
EXPORTED = ("orr_abi_version", "orr_status_string", "orr_traversal_name", "orr_last_error",
            "orr_workspace_bytes", "orr_build_tree", "orr_tree_walk", "orr_tree_walk_grouped",
            "orr_tree_walk_descend", "orr_tree_walk_min_advance", "orr_tree_walk_width", "orr_tree_walk_range",
            "orr_tree_shard_bounds", "orr_eval_forces", "orr_eval_forces_noalloc", "orr_workspace_check", "orr_tree_info_get",
            "orr_tree_check", "orr_tree_export", "orr_tree_export_schedule", "orr_direct_forces",
            "orr_direct_forces_targets", "orr_direct_forces_fp64_targets", "orr_selftest_inv_sqrt", "orr_tree_free")

_lib = None
_vp = ctypes.c_void_p


class OrrError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


class Timings(ctypes.Structure):
    _fields_ = [(f, ctypes.c_float) for f in
                ("cube_keys_ms", "sort_ms", "gather_ms", "build_ms", "moments_ms", "walk_ms", "scatter_ms",
                 "total_ms")]

    def as_dict(self):
        return {f: float(getattr(self, f)) for f, _ in self._fields_}


class TreeInfo(ctypes.Structure):
    _fields_ = [("n", ctypes.c_uint32), ("n_nodes", ctypes.c_uint32), ("n_leaves", ctypes.c_uint32),
                ("depth", ctypes.c_uint32), ("max_leaf_count", ctypes.c_uint32), ("leaf_cap", ctypes.c_int32),
                ("lo", ctypes.c_float * 3), ("side", ctypes.c_float), ("input_status", ctypes.c_int32)]


def lib() -> ctypes.CDLL:
    """Load liborr.so; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise OrrError(ORR_ERR_HIP, f"{LIB_PATH} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        i64, i32, f32, sz = ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
        L.orr_abi_version.restype = ctypes.c_int
        L.orr_status_string.argtypes = [ctypes.c_int]
        L.orr_status_string.restype = ctypes.c_char_p
        L.orr_traversal_name.argtypes = [ctypes.c_int]
        L.orr_traversal_name.restype = ctypes.c_char_p
        L.orr_last_error.restype = ctypes.c_char_p
        L.orr_workspace_bytes.argtypes = [i64, i32]
        L.orr_workspace_bytes.restype = sz
        L.orr_build_tree.argtypes = [_vp, _vp, i64, i32, _vp, sz, _vp, ctypes.POINTER(_vp)]
        L.orr_tree_walk.argtypes = [_vp, f32, f32, ctypes.c_int, _vp, _vp, _vp, _vp, _vp, ctypes.POINTER(Timings)]
        L.orr_tree_walk_grouped.argtypes = [_vp, f32, f32, i32, _vp, _vp, _vp, _vp, _vp]
        L.orr_tree_walk_descend.argtypes = [_vp, f32, f32, i32, _vp, _vp, _vp, _vp, _vp]
        L.orr_tree_walk_min_advance.argtypes = [_vp, f32, f32, _vp, _vp, _vp, _vp, _vp]
        L.orr_tree_walk_width.argtypes = [_vp, f32, f32, i32, _vp, _vp, _vp, _vp, _vp]
        L.orr_tree_walk_range.argtypes = [_vp, f32, f32, ctypes.c_int, i64, i64, _vp, _vp, _vp, _vp, _vp]
        L.orr_tree_shard_bounds.argtypes = [_vp, i32, ctypes.POINTER(i64)]
        L.orr_eval_forces.argtypes = [_vp, _vp, i64, f32, f32, i32, ctypes.c_int, _vp, _vp, _vp, _vp, _vp, _vp, sz,
                                      _vp, ctypes.POINTER(Timings)]
        L.orr_eval_forces_noalloc.argtypes = [_vp, _vp, i64, f32, f32, i32, ctypes.c_int, _vp, _vp, _vp, _vp,
                                              _vp, _vp]
        L.orr_workspace_check.argtypes = [_vp, sz, _vp]
        L.orr_tree_info_get.argtypes = [_vp, ctypes.POINTER(TreeInfo)]
        L.orr_tree_check.argtypes = [_vp]
        L.orr_tree_export.argtypes = [_vp] * 9
        L.orr_tree_export_schedule.argtypes = [_vp] * 3
        L.orr_direct_forces.argtypes = [_vp, _vp, i64, f32, _vp, _vp]
        L.orr_direct_forces_targets.argtypes = [_vp, _vp, i64, f32, _vp, i64, _vp, _vp]
        L.orr_direct_forces_fp64_targets.argtypes = [_vp, _vp, i64, ctypes.c_double, _vp, i64, _vp, _vp]
        L.orr_selftest_inv_sqrt.argtypes = [ctypes.c_uint32, ctypes.c_uint32, _vp, _vp, _vp]
        L.orr_tree_free.argtypes = [_vp]
        L.orr_tree_free.restype = None
        for name in ("orr_build_tree", "orr_tree_walk", "orr_tree_walk_grouped", "orr_tree_walk_descend",
                     "orr_tree_walk_min_advance", "orr_tree_walk_width", "orr_tree_walk_range",
                     "orr_tree_shard_bounds", "orr_eval_forces", "orr_eval_forces_noalloc", "orr_workspace_check",
                     "orr_tree_info_get", "orr_tree_check", "orr_tree_export", "orr_tree_export_schedule",
                     "orr_direct_forces",
                     "orr_direct_forces_targets", "orr_direct_forces_fp64_targets", "orr_selftest_inv_sqrt"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def _check(status: int):
    if status != ORR_OK:
        raise OrrError(status, lib().orr_last_error().decode())


def abi_version() -> int:
    return lib().orr_abi_version()


def workspace_bytes(n: int, leaf_cap: int = 32) -> int:
    return int(lib().orr_workspace_bytes(n, leaf_cap))


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(device):
    return torch.cuda.current_stream(device).cuda_stream


def _as_inputs(pos, mass):
    if not (pos.is_cuda and mass.is_cuda):
        raise OrrError(ORR_ERR_INVALID_ARG, "pos and mass must be GPU tensors")
    if pos.dtype != torch.float32 or mass.dtype != torch.float32:
        raise OrrError(ORR_ERR_INVALID_ARG, "pos and mass must be float32")
    if pos.dim() != 2 or pos.shape[1] != 3 or mass.shape != (pos.shape[0],):
        raise OrrError(ORR_ERR_INVALID_ARG, "pos must be [n, 3] and mass [n]")
    return pos.contiguous(), mass.contiguous()


def _device_tensor(t, name, dtype, shape, device):
    """t as the kernels will write it: a contiguous tensor of this dtype and
    shape in the memory of `device`. The C ABI takes bare device pointers and
    cannot check them; a host tensor or a short one here would be a bad
    device address."""
    if not isinstance(t, torch.Tensor) or not t.is_cuda or t.device != device:
        raise OrrError(ORR_ERR_INVALID_ARG, f"{name} must be a tensor on {device}")
    if t.dtype != dtype or tuple(t.shape) != tuple(shape):
        raise OrrError(ORR_ERR_INVALID_ARG, f"{name} must be {dtype} of shape {tuple(shape)}, got {t.dtype} "
                                            f"{tuple(t.shape)}")
    if not t.is_contiguous():
        raise OrrError(ORR_ERR_INVALID_ARG, f"{name} must be contiguous")
    return t


def _workspace(workspace, n, leaf_cap, device):
    """(tensor, bytes): a caller's workspace, checked to lie contiguous on
    `device`, or a new one."""
    if workspace is None:
        workspace = new_workspace(n, leaf_cap, device)
    if not isinstance(workspace, torch.Tensor) or not workspace.is_cuda or workspace.device != device:
        raise OrrError(ORR_ERR_INVALID_ARG, f"workspace must be a tensor on {device}")
    if not workspace.is_contiguous():
        raise OrrError(ORR_ERR_INVALID_ARG, "workspace must be contiguous")
    return workspace, workspace.numel() * workspace.element_size()


def new_workspace(n: int, leaf_cap: int, device) -> torch.Tensor:
    nbytes = workspace_bytes(n, leaf_cap)
    if nbytes == 0:
        raise OrrError(ORR_ERR_RANGE, f"no workspace for n={n}, leaf_cap={leaf_cap}")
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


@dataclass
class Result:
    acc: torch.Tensor             # [n, 3] float32, caller order
    visits_own: torch.Tensor      # [n] int32 (uint32 bits)
    visits_stepped: torch.Tensor
    n_pp: torch.Tensor
    n_pc: torch.Tensor
    timings: dict | None


def _outputs(n, device, out=None):
    """(acc, [visits_own, visits_stepped, n_pp, n_pc]): new tensors, or the
    caller's `out` in that layout, checked (any entry may be None: that
    output is not written)."""
    if out is None:
        acc = torch.empty((n, 3), dtype=torch.float32, device=device)
        cnt = [torch.empty(n, dtype=torch.int32, device=device) for _ in range(4)]
        return acc, cnt
    acc, cnt = out
    if len(cnt) != 4:
        raise OrrError(ORR_ERR_INVALID_ARG, "out must be (acc, [visits_own, visits_stepped, n_pp, n_pc])")
    acc = None if acc is None else _device_tensor(acc, "acc", torch.float32, (n, 3), device)
    cnt = [None if c is None else _device_tensor(c, f"counter {k}", torch.int32, (n,), device)
           for k, c in enumerate(cnt)]
    return acc, cnt


def orr_eval_forces(pos, mass, *, eps=0.05, theta=0.5, leaf_cap=32, traversal="coherent", workspace=None,
                    out=None, timings=False) -> Result:
    """Build the tree and walk it (orr_eval_forces). Counters are returned as
    int32 tensors holding the uint32 values."""
    pos, mass = _as_inputs(pos, mass)
    n = pos.shape[0]
    workspace, ws_bytes = _workspace(workspace, n, leaf_cap, pos.device)
    acc, cnt = _outputs(n, pos.device, out)
    tm = Timings() if timings else None
    st = lib().orr_eval_forces(_ptr(pos), _ptr(mass), n, eps, theta, leaf_cap, TRAVERSALS[traversal],
                               _ptr(acc), *[_ptr(c) for c in cnt], _ptr(workspace), ws_bytes,
                               _stream(pos.device), ctypes.byref(tm) if tm is not None else None)
    _check(st)
    return Result(acc, cnt[0], cnt[1], cnt[2], cnt[3], tm.as_dict() if tm is not None else None)


def orr_eval_forces_noalloc(pos, mass, *, eps=0.05, theta=0.5, leaf_cap=32, traversal="coherent",
                            out=None) -> Result:
    """orr_eval_forces with the library's fixed per-GPU workspace
    (orr_eval_forces_noalloc): allocates no device memory itself; outputs are
    allocated here only when `out` is not given."""
    pos, mass = _as_inputs(pos, mass)
    n = pos.shape[0]
    acc, cnt = _outputs(n, pos.device, out)
    _check(lib().orr_eval_forces_noalloc(_ptr(pos), _ptr(mass), n, eps, theta, leaf_cap, TRAVERSALS[traversal],
                                         _ptr(acc), *[_ptr(c) for c in cnt], _stream(pos.device)))
    return Result(acc, cnt[0], cnt[1], cnt[2], cnt[3], None)


def orr_workspace_check(workspace: torch.Tensor) -> None:
    """Raise if the most recent evaluation in this workspace had non-finite
    input or an invalid sort (orr_workspace_check); synchronises the current
    stream."""
    if not isinstance(workspace, torch.Tensor) or not workspace.is_cuda or not workspace.is_contiguous():
        raise OrrError(ORR_ERR_INVALID_ARG, "workspace must be a contiguous GPU tensor")
    _check(lib().orr_workspace_check(_ptr(workspace), workspace.numel() * workspace.element_size(),
                                     _stream(workspace.device)))


def orr_direct_forces(pos, mass, *, eps=0.05, out=None) -> torch.Tensor:
    """All-pairs float32 direct sum with the walk's term (orr_direct_forces);
    returns acc [n, 3] in caller order."""
    pos, mass = _as_inputs(pos, mass)
    n = pos.shape[0]
    acc = (torch.empty((n, 3), dtype=torch.float32, device=pos.device) if out is None
           else _device_tensor(out, "out", torch.float32, (n, 3), pos.device))
    _check(lib().orr_direct_forces(_ptr(pos), _ptr(mass), n, eps, _ptr(acc), _stream(pos.device)))
    return acc


def orr_direct_forces_targets(pos, mass, targets, *, eps=0.05, out=None) -> torch.Tensor:
    """The all-pairs float32 direct sum for the caller-order targets (a GPU
    int64 tensor) only (orr_direct_forces_targets); returns acc [len(targets), 3]."""
    pos, mass = _as_inputs(pos, mass)
    if not targets.is_cuda or targets.dtype != torch.int64 or targets.dim() != 1:
        raise OrrError(ORR_ERR_INVALID_ARG, "targets must be a 1-d int64 GPU tensor")
    targets = targets.contiguous()
    m = targets.shape[0]
    acc = (torch.empty((m, 3), dtype=torch.float32, device=pos.device) if out is None
           else _device_tensor(out, "out", torch.float32, (m, 3), pos.device))
    if m == 0:
        return acc
    _check(lib().orr_direct_forces_targets(_ptr(pos), _ptr(mass), pos.shape[0], eps, _ptr(targets), m, _ptr(acc),
                                           _stream(pos.device)))
    return acc


def orr_direct_forces_fp64_targets(pos, mass, targets, *, eps=0.05, out=None) -> torch.Tensor:
    """The compensated float64 direct sum (the accuracy reference) for the
    caller-order targets (a GPU int64 tensor) only
    (orr_direct_forces_fp64_targets); returns float64 acc [len(targets), 3]."""
    pos, mass = _as_inputs(pos, mass)
    if not targets.is_cuda or targets.dtype != torch.int64 or targets.dim() != 1:
        raise OrrError(ORR_ERR_INVALID_ARG, "targets must be a 1-d int64 GPU tensor")
    targets = targets.contiguous()
    m = targets.shape[0]
    acc = (torch.empty((m, 3), dtype=torch.float64, device=pos.device) if out is None
           else _device_tensor(out, "out", torch.float64, (m, 3), pos.device))
    if m == 0:
        return acc
    _check(lib().orr_direct_forces_fp64_targets(_ptr(pos), _ptr(mass), pos.shape[0], float(eps), _ptr(targets), m,
                                                _ptr(acc), _stream(pos.device)))
    return acc


def orr_selftest_inv_sqrt(first_bits: int, last_bits: int, device="cuda"):
    """Compare the walk's inverse square root with the IEEE operations over a
    range of float bit patterns; returns (mismatch count, example bit patterns)."""
    mism = torch.zeros(1, dtype=torch.int64, device=device)
    ex = torch.zeros(8, dtype=torch.int32, device=device)
    _check(lib().orr_selftest_inv_sqrt(first_bits, last_bits, _ptr(mism), _ptr(ex), _stream(torch.device(device))))
    torch.cuda.synchronize(device)
    k = int(mism.item())
    return k, [int(v) & 0xffffffff for v in ex.cpu().tolist()[:min(k, 8)]]


class Tree:
    """A built tree (orr_build_tree); the workspace tensor is kept alive with it."""

    def __init__(self, pos, mass, leaf_cap=32, workspace=None):
        pos, mass = _as_inputs(pos, mass)
        self.n = pos.shape[0]
        self.device = pos.device
        self.workspace, ws_bytes = _workspace(workspace, self.n, leaf_cap, pos.device)
        self._inputs = (pos, mass)
        h = _vp()
        _check(lib().orr_build_tree(_ptr(pos), _ptr(mass), self.n, leaf_cap, _ptr(self.workspace),
                                    ws_bytes, _stream(pos.device), ctypes.byref(h)))
        self._h = h

    def walk(self, eps=0.05, theta=0.5, traversal="coherent", out=None, timings=False) -> Result:
        """The walk of the built tree (orr_tree_walk); timings=True times it
        with HIP events and synchronises."""
        acc, cnt = _outputs(self.n, self.device, out)
        tm = Timings() if timings else None
        _check(lib().orr_tree_walk(self._h, eps, theta, TRAVERSALS[traversal], _ptr(acc),
                                   *[_ptr(c) for c in cnt], ctypes.byref(tm) if tm is not None else None))
        return Result(acc, cnt[0], cnt[1], cnt[2], cnt[3], tm.as_dict() if tm is not None else None)

    def walk_grouped(self, eps=0.05, theta=0.5, group_width=32, out=None) -> Result:
        """The walk with groups of group_width targets sharing a node index
        (orr_tree_walk_grouped)."""
        acc, cnt = _outputs(self.n, self.device, out)
        _check(lib().orr_tree_walk_grouped(self._h, eps, theta, group_width, _ptr(acc), *[_ptr(c) for c in cnt]))
        return Result(acc, cnt[0], cnt[1], cnt[2], cnt[3], None)

    def walk_descend(self, eps=0.05, theta=0.5, group_width=64, out=None) -> Result:
        """The descend-together group walk (orr_tree_walk_descend)."""
        acc, cnt = _outputs(self.n, self.device, out)
        _check(lib().orr_tree_walk_descend(self._h, eps, theta, group_width, _ptr(acc), *[_ptr(c) for c in cnt]))
        return Result(acc, cnt[0], cnt[1], cnt[2], cnt[3], None)

    def walk_min_advance(self, eps=0.05, theta=0.5, out=None) -> Result:
        """The coherent walk advancing by an explicit wave minimum of the
        lanes' next nodes (orr_tree_walk_min_advance); same outputs as the
        coherent walk."""
        acc, cnt = _outputs(self.n, self.device, out)
        _check(lib().orr_tree_walk_min_advance(self._h, eps, theta, _ptr(acc), *[_ptr(c) for c in cnt]))
        return Result(acc, cnt[0], cnt[1], cnt[2], cnt[3], None)

    def walk_width(self, eps=0.05, theta=0.5, width=64, out=None) -> Result:
        """The coherent walk at coherence width 32, 64, 128 or 256 with the
        production machinery (orr_tree_walk_width)."""
        acc, cnt = _outputs(self.n, self.device, out)
        _check(lib().orr_tree_walk_width(self._h, eps, theta, width, _ptr(acc), *[_ptr(c) for c in cnt]))
        return Result(acc, cnt[0], cnt[1], cnt[2], cnt[3], None)

    def walk_range(self, first, count, eps=0.05, theta=0.5, traversal="coherent", out=None) -> Result:
        """The walk of the sorted targets [first, first + count), whole waves
        (orr_tree_walk_range); writes only those targets' outputs."""
        acc, cnt = _outputs(self.n, self.device, out)
        _check(lib().orr_tree_walk_range(self._h, eps, theta, TRAVERSALS[traversal], first, count, _ptr(acc),
                                         *[_ptr(c) for c in cnt]))
        return Result(acc, cnt[0], cnt[1], cnt[2], cnt[3], None)

    def shard_bounds(self, k: int) -> list:
        """k + 1 bounds of contiguous target ranges of nearly equal estimated
        walk cost (orr_tree_shard_bounds); synchronises the stream."""
        b = (ctypes.c_int64 * (k + 1))()
        _check(lib().orr_tree_shard_bounds(self._h, k, b))
        return list(b)

    def info(self) -> dict:
        ti = TreeInfo()
        st = lib().orr_tree_info_get(self._h, ctypes.byref(ti))
        if st not in (ORR_OK, ORR_ERR_NONFINITE):
            _check(st)
        return {"n": ti.n, "n_nodes": ti.n_nodes, "n_leaves": ti.n_leaves, "depth": ti.depth,
                "max_leaf_count": ti.max_leaf_count, "leaf_cap": ti.leaf_cap, "lo": list(ti.lo),
                "side": ti.side, "input_status": ti.input_status}

    def check(self):
        _check(lib().orr_tree_check(self._h))

    def export(self) -> dict:
        nn = self.info()["n_nodes"]
        d = self.device
        out = {"keys_sorted": torch.empty(self.n, dtype=torch.int64, device=d),
               "perm": torch.empty(self.n, dtype=torch.int32, device=d),
               "level": torch.empty(nn, dtype=torch.uint8, device=d),
               "begin": torch.empty(nn, dtype=torch.int32, device=d),
               "count": torch.empty(nn, dtype=torch.int32, device=d),
               "escape": torch.empty(nn, dtype=torch.int32, device=d),
               "geom": torch.empty((nn, 4), dtype=torch.float32, device=d),
               "s2": torch.empty(nn, dtype=torch.float32, device=d)}
        _check(lib().orr_tree_export(self._h, *[_ptr(out[k]) for k in
                                                ("keys_sorted", "perm", "level", "begin", "count", "escape",
                                                 "geom", "s2")]))
        return out

    def export_schedule(self) -> dict:
        """The coherent walk's schedule: wave costs and the eight XCD lists."""
        nw = (self.n + 63) // 64
        out = {"wave_cost": torch.empty(nw, dtype=torch.int32, device=self.device),
               "order": torch.empty(64 * ((nw + 63) // 64) + 8, dtype=torch.int32, device=self.device)}
        _check(lib().orr_tree_export_schedule(self._h, _ptr(out["wave_cost"]), _ptr(out["order"])))
        return out

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and _lib is not None:
            _lib.orr_tree_free(h)
            self._h = None
