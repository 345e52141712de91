"""AddressSanitizer and UndefinedBehaviorSanitizer runs of the host code (the
performance page's "A note on the sanitisers" keeps the sanitisers on every
translation unit they can build; here that is all host code, never device
code):

- the oracle (plain C) built with both sanitizers and its pins run against
  that build, in a child process with the sanitizer runtimes preloaded;
- liborr's host code (argument checks, workspace layout, error paths) built
  with both sanitizers through -Xarch_host, driven by a C program that
  reaches every entry point's rejection and fault-injection paths without a
  GPU (tests/sanitize_abi_driver.c).

Any sanitizer report aborts the child and fails the test. CPU only."""

import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]
ENV_SAN = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1:detect_odr_violation=0",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}

pytestmark = pytest.mark.slow


def _gcc_runtime(name):
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_pins_under_asan_and_ubsan(tmp_path):
    sys.path.insert(0, ROOT)
    from oracle import build as oracle_build

    asan, ubsan = _gcc_runtime("libasan.so"), _gcc_runtime("libubsan.so")
    if not (asan and ubsan):
        pytest.skip("gcc sanitizer runtimes not installed")
    lib = str(tmp_path / "liborr_oracle_san.so")
    oracle_build.build(SAN, out=lib)
    env = dict(os.environ, ORR_ORACLE_LIB=lib, LD_PRELOAD=f"{asan}:{ubsan}", **ENV_SAN)
    pins = sorted(glob.glob(os.path.join(ROOT, "tests", "test_oracle_*.py")))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not slow",
                        "-k", "not 65536", *pins], cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr


def test_abi_host_code_under_asan_and_ubsan(tmp_path):
    sys.path.insert(0, ROOT)
    from barnes_hut_gravitational_amd import build_lib

    clang = "/opt/rocm/llvm/bin/clang"
    if not (os.path.exists(build_lib.HIPCC) and os.path.exists(clang)):
        pytest.skip("ROCm toolchain not available")
    out = str(tmp_path / "liborr_san.so")
    host_san = []
    for f in SAN[:2] + SAN[2:]:
        host_san += ["-Xarch_host", f]
    # objects with host-side sanitizers; device code is built as in the product
    objs = [build_lib._compile(src, host_san, str(tmp_path)) for src in build_lib.SOURCES]
    link = [clang + "++", "-shared", "-fPIC", *objs, "-o", out, "-fsanitize=address,undefined", "-shared-libasan",
            "-L/opt/rocm/lib", "-lamdhip64", *build_lib.LINK_LIBS]
    # the objects' device code needs nothing more: it is embedded as built
    subprocess.run(link, check=True, capture_output=True, text=True)
    rt = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    if not rt:
        pytest.skip("clang AddressSanitizer runtime not installed")
    drv = str(tmp_path / "abi_driver")
    subprocess.run([clang, *SAN, "-shared-libasan", "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "sanitize_abi_driver.c"), out, "-o", drv,
                    f"-Wl,-rpath,{tmp_path}:{os.path.dirname(rt[0])}"], check=True, capture_output=True, text=True)
    env = dict(os.environ, **ENV_SAN)
    env.pop("ORR_FAULT_INJECT", None)
    r = subprocess.run([drv], env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "abi driver ok" in r.stdout
