"""Build liborr.so (HIP, gfx950) in-tree: barnes_hut_gravitational_amd/liborr.so,
and its checked build liborr_checked.so (ORR_CHECKED=1: every index a kernel
takes from device data is tested against its array's length, and a failure is
reported instead of read or written; csrc/checked.h).

Every translation unit is compiled by hipcc for gfx950 with
  -ffp-contract=off   no fused multiply-add contraction: every float step is
                      one correctly rounded operation, as the ABI promises;
  -packed-fp32-ops    disabled: no packed FP32 instructions are generated.
Objects go to _build/ (git-ignored); the library is linked next to this file.
"""

from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "liborr.so")
CHECKED_LIB = os.path.join(PKG, "liborr_checked.so")
SOURCES = ["cube_keys.hip", "sort.hip", "tree.hip", "walk.hip", "walk_grouped.hip", "walk_width.hip", "direct.hip", "orr_api.hip"]
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", INCLUDE, "-I", CSRC, "-Wall", "-Wno-unused-function"]
# Libraries the host code links: roctx, for the phase ranges that rocprofv3
# --marker-trace shows.
LINK_LIBS = ["-L/opt/rocm/lib", "-lrocprofiler-sdk-roctx", "-Wl,-rpath,/opt/rocm/lib"]


def _compile(src: str, extra=(), build_dir=BUILD) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{msg}")
    if msg.strip():
        print(msg, file=sys.stderr)
    return obj


def build(jobs: int = 8, extra_flags=(), out: str = LIB, build_dir: str | None = None) -> str:
    """Compile and link; extra_flags (e.g. -D definitions) and out allow
    variant builds elsewhere."""
    if build_dir is None:
        build_dir = BUILD if out == LIB else out + ".objs"
    os.makedirs(build_dir, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(jobs, len(SOURCES))) as ex:
        objs = list(ex.map(lambda src: _compile(src, extra_flags, build_dir), SOURCES))
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, *LINK_LIBS, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, out)
    return out


def build_checked(jobs: int = 8) -> str:
    """The checked build, liborr_checked.so (same ABI)."""
    return build(jobs, ["-DORR_CHECKED=1"], CHECKED_LIB, os.path.join(BUILD, "checked"))


def resources(src: str = "walk.hip") -> list:
    """Per-kernel resources the compiler gives one source's gfx950 code:
    (kernel, VGPRs, SGPRs, LDS bytes, scratch bytes per lane, VGPR spills),
    from the code object metadata of a device-only assembly build."""
    import re
    import tempfile

    with tempfile.TemporaryDirectory() as d:
        asm = os.path.join(d, "k.s")
        cmd = [HIPCC, *FLAGS, "--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", asm]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
        text = open(asm).read()
    meta = text[text.index("amdhsa.kernels:"):]
    out = []
    for blk in meta.split("  - .agpr_count")[1:]:
        def field(k):
            return re.search(r"\." + k + r":\s+(\S+)", blk).group(1)
        out.append((field("name"), int(field("vgpr_count")), int(field("sgpr_count")),
                    int(field("group_segment_fixed_size")), int(field("private_segment_fixed_size")),
                    int(field("vgpr_spill_count"))))
    return out


if __name__ == "__main__":
    if len(sys.argv) > 1 and sys.argv[1] == "--resources":
        for src in sys.argv[2:] or ["walk.hip"]:
            for name, v, sg, lds, scratch, spill in resources(src):
                print(f"{src}\t{name}\tvgpr {v}\tsgpr {sg}\tlds {lds}\tscratch {scratch}\tvgpr_spill {spill}")
    else:
        print(build())
        print(build_checked())
