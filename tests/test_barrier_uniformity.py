"""Barriers only in uniform control flow, checked in the generated code.

A work-group barrier inside a loop that some lanes of a wave can leave while
others stay is a miscompile waiting to happen: the compiler runs such a loop
with an execution mask, and a lane that has left still reaches the barrier
through the other lanes' iterations. The kernels keep every loop that holds a
barrier under bounds the compiler can prove uniform (values read with
readfirstlane, or loaded through the scalar unit), and this test checks the
result in the gfx950 assembly of every kernel, for the normal and the checked
build:

* the control-flow graph of each kernel from its branch instructions;
* natural loops from back edges to a dominator (Cooper, Harvey and Kennedy's
  iterative dominator algorithm);
* a loop is divergent when one of its blocks removes lanes from the execution
  mask (s_andn2_b64 exec, exec, ...) and branches out of the loop;
* no divergent loop may contain s_barrier.

The analysis is pinned by two small kernels compiled the same way: the same
loop with a barrier, once with a trip count that differs between lanes
(flagged) and once with a uniform one (not flagged). Nothing here runs on a
GPU; hipcc compiles for gfx950 on the host.
"""

import os
import re
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

from barnes_hut_gravitational_amd import build_lib

BUILDS = {"normal": [], "checked": ["-DORR_CHECKED=1"]}


def device_asm(src_path, extra=()):
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "k.s")
        cmd = [build_lib.HIPCC, *build_lib.FLAGS, *extra, "--cuda-device-only", "-S", src_path, "-o", out]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        return open(out).read()


def kernel_blocks(asm):
    """{kernel name: [(label, [instructions])]} in program order."""
    lines = asm.split("\n")
    functions = set(re.findall(r"\.type\s+(\S+),@function", asm))
    out = {}
    for st, line in enumerate(lines):
        m = re.match(r"^(_Z\w+):\s*(;.*)?$", line)
        if not m or m.group(1) not in functions:
            continue
        name = m.group(1)
        end = next(i for i in range(st, len(lines)) if lines[i].startswith(".Lfunc_end"))
        blocks, cur, lab = [], [], "ENTRY"
        for l in lines[st + 1:end]:
            b = re.match(r"^(\.LBB\d+_\d+|; %bb\.\d+):", l)
            if b:
                blocks.append((lab, cur))
                lab, cur = b.group(1), []
                continue
            t = l.strip()
            if t and not t.startswith((";", ".")):
                cur.append(t)
        blocks.append((lab, cur))
        out[name] = blocks
    return out


def cfg(blocks):
    index = {lab: i for i, (lab, _) in enumerate(blocks)}
    succ = [set() for _ in blocks]
    for i, (_, ins) in enumerate(blocks):
        falls = True
        for t in ins:
            m = re.match(r"(s_cbranch_\w+|s_branch)\s+(\.LBB\d+_\d+)", t)
            if m:
                succ[i].add(index[m.group(2)])
                if m.group(1) == "s_branch":
                    falls = False
            if t.startswith("s_endpgm"):
                falls = False
        if falls and i + 1 < len(blocks):
            succ[i].add(i + 1)
    pred = [set() for _ in blocks]
    for i, ss in enumerate(succ):
        for j in ss:
            pred[j].add(i)
    return succ, pred


def immediate_dominators(succ, pred):
    """{block: immediate dominator} for every block reachable from block 0."""
    seen, post, stack = {0}, [], [(0, iter(sorted(succ[0])))]
    while stack:
        v, it = stack[-1]
        for w in it:
            if w not in seen:
                seen.add(w)
                stack.append((w, iter(sorted(succ[w]))))
                break
        else:
            stack.pop()
            post.append(v)
    rpo = post[::-1]
    num = {v: k for k, v in enumerate(rpo)}
    idom = {0: 0}
    changed = True
    while changed:
        changed = False
        for v in rpo[1:]:
            ps = [p for p in pred[v] if p in idom]
            new = ps[0]
            for p in ps[1:]:
                a, b = p, new
                while a != b:
                    while num[a] > num[b]:
                        a = idom[a]
                    while num[b] > num[a]:
                        b = idom[b]
                new = a
            if idom.get(v) != new:
                idom[v] = new
                changed = True
    return idom


def dominates(h, u, idom):
    while u != h:
        if idom[u] == u:
            return False
        u = idom[u]
    return True


def divergent_barrier_loops(blocks):
    """Labels of the headers of divergent loops that contain s_barrier."""
    succ, pred = cfg(blocks)
    idom = immediate_dominators(succ, pred)
    found = []
    for u in idom:
        for h in succ[u]:
            if h not in idom or not dominates(h, u, idom):
                continue
            body, stack = {h, u}, ([u] if u != h else [])
            while stack:
                x = stack.pop()
                for p in pred[x]:
                    if p not in body and p in idom:
                        body.add(p)
                        stack.append(p)
            lanes_leave = any(any(t.startswith("s_andn2_b64 exec, exec") for t in blocks[b][1]) and succ[b] - body
                              for b in body)
            barrier = any(any(t.startswith("s_barrier") for t in blocks[b][1]) for b in body)
            if lanes_leave and barrier:
                found.append(blocks[h][0])
    return found


PIN = r"""
#include <hip/hip_runtime.h>
namespace orr_pin {
__global__ __launch_bounds__(256) void k_lane_bound(int *out, const int *in) {
    __shared__ int s[256];
    int acc = 0;
    const int n = in[threadIdx.x];  // differs between lanes
    for (int i = 0; i < n; i++) {
        s[threadIdx.x] = acc + i;
        __syncthreads();
        acc += s[(threadIdx.x + 1) & 255];
        __syncthreads();
    }
    out[threadIdx.x] = acc;
}
__global__ __launch_bounds__(256) void k_uniform_bound(int *out, const int *in) {
    __shared__ int s[256];
    int acc = 0;
    const int n = __builtin_amdgcn_readfirstlane(in[threadIdx.x]);  // one value for the wave
    for (int i = 0; i < n; i++) {
        s[threadIdx.x] = acc + i;
        __syncthreads();
        acc += s[(threadIdx.x + 1) & 255];
        __syncthreads();
    }
    out[threadIdx.x] = acc;
}
}
"""


def test_analysis_flags_a_barrier_in_a_divergent_loop():
    with tempfile.TemporaryDirectory() as d:
        src = os.path.join(d, "pin.hip")
        open(src, "w").write(PIN)
        kernels = kernel_blocks(device_asm(src))
    bad = [k for k in kernels if "k_lane_bound" in k]
    good = [k for k in kernels if "k_uniform_bound" in k]
    assert len(bad) == 1 and len(good) == 1
    assert divergent_barrier_loops(kernels[bad[0]])
    assert not divergent_barrier_loops(kernels[good[0]])


@pytest.fixture(scope="module")
def library_asm():
    jobs = [(src, build) for build in BUILDS for src in build_lib.SOURCES]
    with ThreadPoolExecutor(max_workers=8) as ex:
        texts = list(ex.map(lambda j: device_asm(os.path.join(build_lib.CSRC, j[0]), BUILDS[j[1]]), jobs))
    return dict(zip(jobs, texts))


@pytest.mark.parametrize("build", sorted(BUILDS))
def test_no_barrier_in_a_divergent_loop(library_asm, build):
    checked = 0
    problems = []
    for (src, b), asm in library_asm.items():
        if b != build:
            continue
        for name, blocks in kernel_blocks(asm).items():
            checked += 1
            loops = divergent_barrier_loops(blocks)
            if loops:
                problems.append(f"{src} {name}: {loops[:4]}")
    assert checked >= 30, checked
    assert not problems, problems
