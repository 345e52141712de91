"""CPU tests of the C ABI's error paths through its fault-injection hook
(environment variable ORR_FAULT_INJECT names a site that then reports a
failure instead of calling HIP or allocating): every entry point returns the
documented status with a message naming the site, and nothing aborts. Valid
arguments with placeholder device pointers are used; the injected site is
the first device work each call reaches, so no GPU is touched."""

import ctypes
import os

import pytest

from barnes_hut_gravitational_amd import orr

WS = 256  # a 256-byte aligned placeholder workspace address; never dereferenced here


@pytest.fixture
def inject(monkeypatch):
    def set_site(site):
        monkeypatch.setenv("ORR_FAULT_INJECT", site)
    yield set_site
    monkeypatch.delenv("ORR_FAULT_INJECT", raising=False)


def eval_forces(timings=False):
    L = orr.lib()
    tm = orr.Timings()
    st = L.orr_eval_forces(1, 1, 1000, 0.05, 0.5, 32, 1, None, None, None, None, None, WS, 1 << 30, None,
                           ctypes.byref(tm) if timings else None)
    return st, L.orr_last_error().decode()


@pytest.mark.parametrize("site,where", [("cube", "root cube"), ("events", "hipEventCreate")])
def test_eval_forces_reports_injected_fault(inject, site, where):
    inject(site)
    st, msg = eval_forces(timings=site == "events")
    assert st == orr.ORR_ERR_HIP and where in msg, msg


def test_build_tree_reports_host_allocation_failure(inject):
    inject("alloc")
    L = orr.lib()
    h = ctypes.c_void_p(12345)
    st = L.orr_build_tree(1, 1, 1000, 32, WS, 1 << 30, None, ctypes.byref(h))
    assert st == orr.ORR_ERR_HOST_MEMORY and h.value is None
    assert L.orr_last_error() == b"host allocation failed"
    assert L.orr_status_string(orr.ORR_ERR_HOST_MEMORY) == b"host allocation failed"


def test_build_tree_reports_first_launch(inject):
    inject("cube")
    L = orr.lib()
    h = ctypes.c_void_p()
    assert L.orr_build_tree(1, 1, 1000, 32, WS, 1 << 30, None, ctypes.byref(h)) == orr.ORR_ERR_HIP
    assert h.value is None and b"root cube" in L.orr_last_error()


def test_noalloc_reports_scratch_setup_failure(inject):
    inject("scratch")
    L = orr.lib()
    st = L.orr_eval_forces_noalloc(1, 1, 1000, 0.05, 0.5, 32, 1, None, None, None, None, None, None)
    assert st == orr.ORR_ERR_HIP and b"hipGetDevice" in L.orr_last_error()


def test_direct_sums_report_injected_fault(inject):
    inject("direct")
    L = orr.lib()
    assert L.orr_direct_forces(1, 1, 100, 0.05, 1, None) == orr.ORR_ERR_HIP
    assert b"direct sum" in L.orr_last_error()
    assert L.orr_direct_forces_targets(1, 1, 100, 0.05, 1, 10, 1, None) == orr.ORR_ERR_HIP
    assert L.orr_direct_forces_fp64_targets(1, 1, 100, 0.05, 1, 10, 1, None) == orr.ORR_ERR_HIP


def test_workspace_check_reports_sync_failure(inject):
    inject("sync")
    L = orr.lib()
    assert L.orr_workspace_check(WS, 1 << 20, None) == orr.ORR_ERR_HIP
    assert b"injected" in L.orr_last_error()


def test_other_site_names_leave_the_checks_in_place(inject):
    """An unknown site injects nothing: argument checks still come first."""
    inject("no-such-site")
    L = orr.lib()
    assert L.orr_eval_forces(1, 1, 0, 0.05, 0.5, 32, 1, None, None, None, None, None, WS, 1 << 30, None,
                             None) == orr.ORR_ERR_RANGE
    assert "ORR_FAULT_INJECT" in os.environ
