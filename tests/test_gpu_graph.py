"""The evaluation under HIP graph capture: orr_eval_forces enqueues only
kernels on the caller's stream (no allocation, copy, fill or host wait when
timings are off), so a captured evaluation replays to the eager result. The
graph is replayed several times with eager evaluations of other inputs and
host synchronisations in between, and every replay is compared with the
eager outputs bit for bit."""

import pytest
import torch

from barnes_hut_gravitational_amd import inputs, orr

from parity import to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    orr.lib()


@pytest.mark.parametrize("traversal", ["coherent", "independent"])
def test_eval_forces_graph_replays(traversal):
    pos, mass = inputs.make("plummer", 20000)
    P, M = to_dev(pos, mass)
    n = len(mass)
    ws = orr.new_workspace(n, 32, "cuda")
    out = orr._outputs(n, "cuda")
    ref = orr.orr_eval_forces(P, M, traversal=traversal, workspace=ws)
    torch.cuda.synchronize()
    ref = [ref.acc.clone(), ref.visits_own.clone(), ref.visits_stepped.clone(), ref.n_pp.clone(), ref.n_pc.clone()]
    # other work between replays: another evaluation with its own workspace
    pos2, mass2 = inputs.make("uniform", 5000)
    P2, M2 = to_dev(pos2, mass2)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        orr.orr_eval_forces(P, M, traversal=traversal, workspace=ws, out=out)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        orr.orr_eval_forces(P, M, traversal=traversal, workspace=ws, out=out)
    for replay in range(4):
        print(f"[case] graph replay {replay} traversal={traversal}", flush=True)
        out[0].fill_(float("nan"))
        for c in out[1]:
            c.fill_(-1)
        g.replay()
        torch.cuda.synchronize()
        got = [out[0], *out[1]]
        for a, b in zip(got, ref):
            assert torch.equal(a.view(torch.int32), b.view(torch.int32))
        orr.orr_eval_forces(P2, M2, traversal=traversal)  # eager work in between
        torch.cuda.synchronize()
