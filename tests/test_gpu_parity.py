"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Integer work (keys, order, topology, escape indices, node records, per-target
interaction and visit counts) must match bit for bit; float32 accelerations
within 1e-5 max relative per-particle error, and, by construction of the
term's operation sequence, bit for bit. The two traversals must agree with
each other exactly (ADR-0029, Consequences).
"""

import os
import re

import numpy as np
import pytest
import torch

import oracle
from barnes_hut_gravitational_amd import inputs, orr

from eps_bound import smallest_eps
from parity import check_acc_bitwise, check_tree, check_walk, to_dev, u32

pytestmark = pytest.mark.gpu
EPS, THETA = inputs.EPS, inputs.THETA


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    orr.lib()


def run_full_case(pos, mass, cap, eps, theta):
    print(f"[case] n={len(mass)} cap={cap} eps={eps} theta={theta}", flush=True)
    ref = oracle.evaluate(pos, mass, eps, theta, cap)
    P, M = to_dev(pos, mass)
    tree = orr.Tree(P, M, cap)
    check_tree(tree, ref.tree)
    res = {}
    for tr in ("coherent", "independent"):
        r = tree.walk(eps, theta, tr)
        torch.cuda.synchronize()
        check_walk(r, ref, tr)
        check_acc_bitwise(r, ref.acc)
        res[tr] = r
    a, b = res["coherent"], res["independent"]
    assert torch.equal(a.acc.view(torch.int32), b.acc.view(torch.int32))
    for f in ("visits_own", "n_pp", "n_pc"):
        assert torch.equal(getattr(a, f), getattr(b, f))
    return ref, res


SMALL = [("plummer", n, 32, 0.5) for n in (1, 2, 3, 31, 32, 33, 63, 64, 65, 100, 257, 1000, 4097)] + [
    ("plummer", 2000, 1, 0.5), ("plummer", 2000, 8, 0.0), ("plummer", 3000, 256, 0.5), ("merger", 5000, 16, 0.7),
    ("uniform", 6000, 32, 0.3), ("plummer", 4096, 32, 1.0), ("merger", 2048, 3, 100.0)]


@pytest.mark.parametrize("kind,n,cap,theta", SMALL)
def test_small_cases(kind, n, cap, theta):
    pos, mass = inputs.make(kind, n)
    run_full_case(pos, mass, cap, EPS, theta)


def test_inverse_sqrt_exhaustive():
    """The walk's shorter inverse square root equals the IEEE square root then
    division for every float in its domain [2^-96, +inf]."""
    first, last = 0x0F800000, 0x7F800000  # 2^-96 .. +inf
    k, ex = orr.orr_selftest_inv_sqrt(first, last)
    assert k == 0, [hex(v) for v in ex]


def test_smallest_admitted_eps_and_rejected_tiny_eps():
    """At the smallest admitted eps (the own term's eps^-3 just below FLT_MAX)
    every output is finite and the oracle's; just below it, and far below,
    both sides reject eps instead of returning NaN."""
    lo, below = smallest_eps()
    pos, mass = inputs.make("plummer", 3000)
    run_full_case(pos, mass, 32, lo, 0.5)
    P, M = to_dev(pos, mass)
    for eps in (below, 1e-20):
        with pytest.raises(orr.OrrError) as e:
            orr.orr_eval_forces(P, M, eps=eps)
        assert e.value.status == orr.ORR_ERR_RANGE
        with pytest.raises(oracle.OracleError):
            oracle.evaluate(pos, mass, eps, 0.5, 32)


def test_unequal_masses_and_small_eps():
    pos, mass = inputs.make("plummer", 3000)
    mass = (mass * np.random.default_rng(2).uniform(0.1, 3.0, 3000)).astype(np.float32)
    mass[::7] = 0.0
    run_full_case(pos, mass, 32, 1e-3, 0.5)


def test_degenerate_inputs():
    # all particles at one point: a chain down to level 21 ending in one big leaf
    run_full_case(np.full((100, 3), 0.25, np.float32), np.full(100, 0.01, np.float32), 32, EPS, 0.5)
    # heavy duplicates on a coarse lattice, over-cap leaves at level 21
    rng = np.random.default_rng(4)
    pos = rng.integers(0, 3, (3000, 3)).astype(np.float32)
    run_full_case(pos, np.full(3000, 1 / 3000, np.float32), 8, EPS, 0.5)
    # collinear, and a flat (zero-extent) axis
    t = np.linspace(-1, 1, 1500, dtype=np.float32)
    run_full_case(np.stack([t, 2 * t, np.zeros_like(t)], 1), np.full(1500, 1 / 1500, np.float32), 32, EPS, 0.5)
    # every mass zero (each node's centre is its first particle), and all the
    # mass on one particle
    pos, mass = inputs.make("plummer", 3000)
    run_full_case(pos, np.zeros(3000, np.float32), 32, EPS, 0.5)
    one = np.zeros(3000, np.float32)
    one[1234] = 1.0
    run_full_case(pos, one, 16, EPS, 0.5)
    # far from the origin: a large corner, few position bits inside the cube
    pos, mass = inputs.make("plummer", 3000)
    run_full_case((pos + np.float32(1e4)).astype(np.float32), mass, 32, EPS, 0.5)
    run_full_case((pos * np.float32(1e-3) - np.float32(7e3)).astype(np.float32), mass, 8, EPS, 0.5)
    # tiny and huge coordinate scales
    pos, mass = inputs.make("plummer", 2000)
    run_full_case(pos * np.float32(1e-30), mass, 32, EPS, 0.5)
    run_full_case(pos * np.float32(1e30), mass, 32, EPS, 0.5)


@pytest.mark.parametrize("kind,n,cap,theta", [("plummer", 4097, 32, 0.5), ("merger", 5000, 16, 0.7),
                                               ("plummer", 131072, 32, 0.5)])
def test_64bit_node_offsets(kind, n, cap, theta, monkeypatch):
    """The coherent walk's large-tree path (node records by 64-bit index,
    taken on its own above about 82 million particles), forced at sizes the
    oracle finishes in seconds."""
    monkeypatch.setenv("ORR_WALK_NODE_OFFSETS", "64")
    pos, mass = inputs.make(kind, n)
    run_full_case(pos, mass, cap, EPS, theta)


def test_64bit_node_offsets_natural_size():
    """The coherent walk's large-tree path taken on its own, not forced. It
    is chosen when the workspace's node bound times 32 bytes passes 4 GiB, and
    at leaf capacity 1 that bound, n + 21 floor(n / 2) + 1, does so above
    11.7 million particles. A ragged uniform cube of 12,000,017 particles:
    the tree bit for bit against the oracle; through the benchmark's entry
    point (orr_eval_forces, coherent), 3,000 sampled targets' accelerations
    and counts against the oracle's walk, and their waves' visits_stepped
    against the oracle's unions; the independent walk equal on every
    target."""
    n, cap = 12_000_017, 1
    assert oracle.max_nodes(n, cap) * 32 > 2**32
    pos, mass = inputs.make("uniform", n)
    print(f"[case] natural 64-bit node offsets n={n} cap={cap}", flush=True)
    ot = oracle.build_tree(pos, mass, cap)
    print(f"[case] oracle tree: {ot.n_nodes} nodes", flush=True)
    P, M = to_dev(pos, mass)
    ws = orr.new_workspace(n, cap, P.device)
    r = orr.orr_eval_forces(P, M, eps=EPS, theta=THETA, leaf_cap=cap, traversal="coherent", workspace=ws,
                            timings=True)
    tg = np.sort(np.random.default_rng(12).choice(n, 3000, replace=False))  # sorted positions
    acc, pp, pc, vis = oracle.walk(ot, EPS, THETA, tg)
    rows = ot.perm[tg].astype(np.int64)  # their caller-order indices
    assert np.array_equal(r.acc.cpu().numpy()[rows].view(np.uint32), acc.view(np.uint32))
    assert np.array_equal(u32(r.n_pp)[rows], pp)
    assert np.array_equal(u32(r.n_pc)[rows], pc)
    assert np.array_equal(u32(r.visits_own)[rows], vis)
    waves, inv = np.unique(tg // 64, return_inverse=True)
    union = oracle.union_visits(ot, EPS, THETA, 64, waves)
    assert np.array_equal(u32(r.visits_stepped)[rows], union[inv])
    tree = orr.Tree(P, M, cap, workspace=ws)
    check_tree(tree, ot)
    ri = tree.walk(EPS, THETA, "independent")
    torch.cuda.synchronize()
    assert torch.equal(r.acc.view(torch.int32), ri.acc.view(torch.int32))
    for f in ("visits_own", "n_pp", "n_pc"):
        assert torch.equal(getattr(r, f), getattr(ri, f))
    print(f"[case] natural 64-bit node offsets ok, timings {r.timings}", flush=True)


@pytest.mark.parametrize("n", [16384, 16385, 32768, 32769, 262144, 262145])
def test_sort_tile_edges(n):
    """The sort's tiles hold 1,024 keys up to 32,768 particles, 2,048 up to
    262,144 and 4,096 above: each size here fills its tiles exactly or leaves a
    last tile of one key, and the three limits switch tile sizes. The
    oracle's tree and walk for Plummer and for heavy duplicates on a lattice
    (long runs of equal keys across tiles, so stability decides the order);
    up to 32,769 particles also for a single point and for a signed-zero
    minimum (the corner must be +0)."""
    pos, mass = inputs.make("plummer", n)
    run_full_case(pos, mass, 32, EPS, 0.5)
    rng = np.random.default_rng(5)
    lat = rng.integers(0, 4, (n, 3)).astype(np.float32)
    run_full_case(lat, np.full(n, 1 / n, np.float32), 8, EPS, 0.5)
    if n > 32769:
        return
    run_full_case(np.full((n, 3), -1.5, np.float32), np.full(n, 1 / n, np.float32), 32, EPS, 0.5)
    z = rng.uniform(0, 1, (n, 3)).astype(np.float32)
    z[::3, 1] = np.float32(-0.0)
    z[1::3, 1] = np.float32(0.0)
    run_full_case(z, np.full(n, 1 / n, np.float32), 32, EPS, 0.5)


def clustered(n_clusters, per, side, seed, outlier=False):
    """n_clusters cubes of edge `side` at random centres in [0.1, 0.9]^3, `per`
    uniform particles each, plus optionally one particle at (3, 3, 3). The
    sort orders keys by their high 32 bits first (a grid of cells 2^-10 to
    2^-11 of the root side) and then each run of equal high bits by the low
    bits: a cube of edge 1e-5 lies in one or a few such cells, so it makes
    runs of up to `per` keys whose low bits mostly differ."""
    rng = np.random.default_rng(seed)
    c = rng.uniform(0.1, 0.9, (n_clusters, 1, 3))
    pos = (c + rng.uniform(0, side, (n_clusters, per, 3))).reshape(-1, 3)
    if outlier:
        pos = np.vstack([pos, [[3.0, 3.0, 3.0]]])
    pos = pos.astype(np.float32)
    return pos, np.full(len(pos), 1 / len(pos), np.float32)


def high_runs(keys):
    """Lengths of the runs of equal high 32 key bits in sorted keys."""
    h = keys >> np.uint64(31)
    starts = np.flatnonzero(np.r_[True, h[1:] != h[:-1]])
    return np.diff(np.r_[starts, len(h)])


@pytest.mark.parametrize("n_clusters,per,side,outlier", [(40, 1500, 1e-5, False), (12, 64, 1e-5, False),
                                                         (9, 65, 1e-5, False), (1, 4096, 1e-5, True),
                                                         (1, 4097, 1e-5, True), (1, 20000, 1e-5, True),
                                                         (3, 30000, 1e-5, False), (2, 9000, 0.0, True),
                                                         (70, 5000, 1e-6, False)])
def test_sort_clustered_runs(n_clusters, per, side, outlier):
    """Runs of equal high key bits of every length class: up to 64 (one
    thread each), 65 to 4,096 (one work-group each), and longer (the
    fallback), at the class limits 64 / 65 and 4,096 / 4,097, with the
    oracle's tree and both walks. Longer runs are sorted by their low bits as
    one array when there are at most 64 of them (here 1, 2 and 3, the 2 of
    them clusters of coincident points whose low bits are all equal) and the
    whole array by the full key otherwise (here 70). The run lengths
    actually produced are printed and their classes asserted."""
    pos, mass = clustered(n_clusters, per, side, 11 + per, outlier)
    ref, _ = run_full_case(pos, mass, 32, EPS, 0.5)
    runs = high_runs(ref.tree.keys_sorted)
    print(f"[runs] max {runs.max()} over 64: {(runs > 64).sum()} over 4096: {(runs > 4096).sum()}", flush=True)
    assert runs.max() > 64 or per <= 64
    if n_clusters == 70:
        assert (runs > 4096).sum() > 64


@pytest.mark.parametrize("n", [1 << 20, 2_000_003])
def test_sort_fallback_large(n):
    """One cluster of n - 1 particles and one far particle: a single run of
    about n keys, sorted by the fallback over hundreds of tiles; the tree
    against the oracle's, bit for bit."""
    pos, mass = clustered(1, n - 1, 1e-5, 3, outlier=True)
    print(f"[case] fallback n={n}", flush=True)
    ot = oracle.build_tree(pos, mass, 32)
    assert high_runs(ot.keys_sorted).max() > 4096
    P, M = to_dev(pos, mass)
    check_tree(orr.Tree(P, M, 32), ot)


@pytest.mark.parametrize("name", ["plummer_16k", "plummer_131k", "uniform_262k"])
def test_configs_full(name):
    pos, mass = inputs.make_config(name)
    ref, _ = run_full_case(pos, mass, inputs.LEAF_CAP, EPS, THETA)
    st = ref.visits_stepped.astype(np.float64).mean() / ref.visits_own.astype(np.float64).mean()
    print(f"[{name}] nodes={ref.tree.n_nodes} visits own {ref.visits_own.mean():.0f} "
          f"stepped {ref.visits_stepped.mean():.0f} redundancy {st:.3f}", flush=True)


@pytest.mark.parametrize("name", ["plummer_1m", "merger_8m"])
def test_configs_large_every_target(name):
    """Full-size workloads in the launch configuration the benchmark times
    (orr_eval_forces, coherent walk): the whole tree bit-exact, and every
    target's acceleration, counts and wave union against the oracle's whole
    evaluation; the independent walk identical to the coherent one."""
    pos, mass = inputs.make_config(name)
    n = len(mass)
    print(f"[case] {name} n={n}", flush=True)
    ref = oracle.evaluate(pos, mass, EPS, THETA, inputs.LEAF_CAP)
    print(f"[{name}] oracle done", flush=True)
    P, M = to_dev(pos, mass)
    ws = orr.new_workspace(n, inputs.LEAF_CAP, P.device)
    r = orr.orr_eval_forces(P, M, eps=EPS, theta=THETA, leaf_cap=inputs.LEAF_CAP, traversal="coherent",
                            workspace=ws, timings=True)
    check_walk(r, ref, "coherent")
    check_acc_bitwise(r, ref.acc)
    tree = orr.Tree(P, M, inputs.LEAF_CAP, workspace=ws)
    check_tree(tree, ref.tree)
    ri = tree.walk(EPS, THETA, "independent")
    torch.cuda.synchronize()
    assert torch.equal(r.acc.view(torch.int32), ri.acc.view(torch.int32))
    for f in ("visits_own", "n_pp", "n_pc"):
        assert torch.equal(getattr(r, f), getattr(ri, f))
    print(f"[{name}] timings {r.timings}", flush=True)


@pytest.mark.parametrize("kind,n", [("plummer", 1000003), ("uniform", 300007), ("merger", 2000001)])
def test_ragged_large_every_target(kind, n):
    """Sizes that are not powers of two at full scale: a last sort tile, a
    last target wave and a last schedule region that are partly empty. The
    tree bit for bit, and every target's acceleration, counts and wave union
    against the oracle's whole evaluation."""
    pos, mass = inputs.make(kind, n)
    print(f"[case] ragged {kind} n={n}", flush=True)
    ref = oracle.evaluate(pos, mass, EPS, THETA, inputs.LEAF_CAP)
    P, M = to_dev(pos, mass)
    r = orr.orr_eval_forces(P, M, eps=EPS, theta=THETA, leaf_cap=inputs.LEAF_CAP, traversal="coherent",
                            timings=True)
    check_walk(r, ref, "coherent")
    check_acc_bitwise(r, ref.acc)
    tree = orr.Tree(P, M, inputs.LEAF_CAP)
    check_tree(tree, ref.tree)


@pytest.mark.parametrize("n", [1000, 20000])
def test_nonfinite_input_reported(n):
    """Non-finite positions and masses and negative masses are flagged, with
    the particle at block 0 of 4 (1,000 particles) or of 79 (20,000) blocks
    of the cube and key kernels."""
    pos, mass = inputs.make("plummer", n)
    for bad_pos, bad_mass in ((np.nan, None), (np.inf, None), (None, -1.0), (None, np.nan)):
        p, m = pos.copy(), mass.copy()
        if bad_pos is not None:
            p[17, 1] = bad_pos
        if bad_mass is not None:
            m[5] = bad_mass
        P, M = to_dev(p, m)
        with pytest.raises(orr.OrrError) as e:
            orr.orr_eval_forces(P, M, timings=True)
        assert e.value.status == orr.ORR_ERR_NONFINITE
        tree = orr.Tree(P, M, 32)
        tree.walk()
        with pytest.raises(orr.OrrError):
            tree.check()
        assert tree.info()["input_status"] == orr.ORR_ERR_NONFINITE
    # the next good input on the same workspace is clean
    P, M = to_dev(pos, mass)
    orr.orr_eval_forces(P, M, timings=True)


def test_workspace_reuse_and_side_stream():
    """A workspace reused for a smaller input, on a non-default stream."""
    big, small = inputs.make("plummer", 20000), inputs.make("uniform", 3000)
    ws = orr.new_workspace(20000, 32, "cuda")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        for pos, mass in (big, small, big):
            ref = oracle.evaluate(pos, mass, EPS, THETA, 32)
            P, M = to_dev(pos, mass)
            r = orr.orr_eval_forces(P, M, workspace=ws)
            s.synchronize()
            check_walk(r, ref, "coherent")


def test_concurrent_streams_separate_workspaces():
    """Evaluations enqueued on four streams at once, each with its own
    workspace and input (sizes that take different team sizes and sort tile
    sizes), several times over without waiting in between: every result is
    bit for bit the oracle's. The library keeps no device state outside the
    caller's workspace."""
    cases = [inputs.make("plummer", 20000), inputs.make("uniform", 70000), inputs.make("merger", 300007),
             clustered(3, 9000, 1e-5, 21)]
    refs = [oracle.evaluate(p, m, EPS, THETA, 32) for p, m in cases]
    dev = [to_dev(p, m) for p, m in cases]
    streams = [torch.cuda.Stream() for _ in cases]
    wss = [orr.new_workspace(len(m), 32, "cuda") for _, m in cases]
    outs = [[None] * 3 for _ in cases]
    torch.cuda.synchronize()
    for rep in range(3):
        for k, (P, M) in enumerate(dev):
            with torch.cuda.stream(streams[k]):
                outs[k][rep] = orr.orr_eval_forces(P, M, workspace=wss[k] if rep != 1 else None)
    torch.cuda.synchronize()
    for k, ref in enumerate(refs):
        for rep in range(3):
            check_walk(outs[k][rep], ref, "coherent")
            check_acc_bitwise(outs[k][rep], ref.acc)
        orr.orr_workspace_check(wss[k])


def test_one_tree_many_walks():
    """A tree built once and walked with different softenings and opening
    angles (including a power-of-two theta^2, which takes the scaled
    comparison, and theta = 0), each walk bit for bit the oracle's for the
    same parameters; the tree itself is unchanged by the walks."""
    pos, mass = inputs.make("merger", 30000)
    ot = oracle.build_tree(pos, mass, 16)
    P, M = to_dev(pos, mass)
    tree = orr.Tree(P, M, 16)
    for eps, theta in ((0.05, 0.5), (0.01, 0.7), (0.2, 0.25), (1e-3, 1.2), (0.05, 0.0)):
        ref, r = oracle.evaluate(pos, mass, eps, theta, 16), tree.walk(eps, theta, "coherent")
        torch.cuda.synchronize()
        print(f"[case] one tree eps={eps} theta={theta}", flush=True)
        check_walk(r, ref, "coherent")
        check_acc_bitwise(r, ref.acc)
    check_tree(tree, ot)


def test_argument_errors_on_device_tensors():
    P, M = to_dev(*inputs.make("plummer", 100))
    for kw in ({"eps": 0.0}, {"eps": float("nan")}, {"theta": -1.0}, {"leaf_cap": 0}, {"leaf_cap": 257}):
        with pytest.raises(orr.OrrError) as e:
            orr.orr_eval_forces(P, M, **kw)
        assert e.value.status == orr.ORR_ERR_RANGE
    with pytest.raises(orr.OrrError) as e:
        orr.orr_eval_forces(P, M, workspace=torch.empty(1024, dtype=torch.uint8, device="cuda"))
    assert e.value.status == orr.ORR_ERR_WORKSPACE
    # Tensors the kernels would write are checked before the call: host
    # memory, wrong shape or dtype, or a strided view would be bad device
    # addresses for the C ABI.
    n = 100
    ws_host = torch.empty(orr.workspace_bytes(n, 32), dtype=torch.uint8)
    acc = torch.empty((n, 3), device="cuda")
    cnt = [torch.empty(n, dtype=torch.int32, device="cuda") for _ in range(4)]
    bad = [dict(workspace=ws_host),
           dict(workspace=torch.empty(2 * orr.workspace_bytes(n, 32), dtype=torch.uint8, device="cuda")[::2]),
           dict(out=(torch.empty((n, 3)), cnt)), dict(out=(torch.empty((n - 1, 3), device="cuda"), cnt)),
           dict(out=(torch.empty((n, 3), dtype=torch.float64, device="cuda"), cnt)),
           dict(out=(torch.empty((3, n), device="cuda").t(), cnt)),
           dict(out=(acc, cnt[:3])), dict(out=(acc, cnt[:3] + [torch.empty(n, dtype=torch.int64, device="cuda")]))]
    for kw in bad:
        with pytest.raises(orr.OrrError) as e:
            orr.orr_eval_forces(P, M, **kw)
        assert e.value.status == orr.ORR_ERR_INVALID_ARG, kw
    tree = orr.Tree(P, M, 32)
    with pytest.raises(orr.OrrError) as e:
        tree.walk(out=(torch.empty((n, 3)), cnt))
    assert e.value.status == orr.ORR_ERR_INVALID_ARG
    with pytest.raises(orr.OrrError) as e:
        orr.orr_direct_forces(P, M, out=torch.empty((n, 3)))
    assert e.value.status == orr.ORR_ERR_INVALID_ARG
    with pytest.raises(orr.OrrError) as e:
        orr.Tree(P, M, 32, workspace=ws_host)
    assert e.value.status == orr.ORR_ERR_INVALID_ARG
    # NULL outputs stay allowed: the library writes only what it is given
    r = orr.orr_eval_forces(P, M, out=(acc, [None, None, cnt[2], None]))
    torch.cuda.synchronize()
    assert r.visits_own is None and torch.isfinite(r.acc).all()


def test_native_library_loaded_once():
    """The in-tree liborr.so is the code that ran, over the same HIP runtime as torch."""
    maps = open("/proc/self/maps").read()
    assert orr.LIB_PATH in maps
    runtimes = {m for m in re.findall(r"(/\S*libamdhip64\.so[.\d]*)", maps)}
    assert len({os.path.realpath(p) for p in runtimes}) == 1, runtimes


@pytest.mark.parametrize("theta", [0.25, 0.125, 2.0 ** -10])
def test_power_of_two_thetas(theta):
    """theta^2 = 2^-e: the coherent walk compares s^2 2^e with d^2 (an
    exponent add on the scalar node record) instead of s^2 with theta^2 d^2;
    the decisions, and so every output, must stay the oracle's."""
    pos, mass = inputs.make("plummer", 3000)
    run_full_case(pos, mass, 16, EPS, theta)


@pytest.mark.parametrize("scale", [2.0 ** -40, 2.0 ** -46, 2.0 ** -48, 2.0 ** 56, 2.0 ** 60])
def test_scaled_compare_range_limits(scale):
    """Coordinate scales on both sides of the range in which every node's
    s^2 2^e is a normal float (the scaled comparison is used inside it, the
    product theta^2 d^2 outside); results are the oracle's either way."""
    pos, mass = inputs.make("plummer", 2000)
    run_full_case((pos * np.float32(scale)).astype(np.float32), mass, 32, EPS, 0.5)
