"""Dispatch order of workgroups over the XCDs, through the test probe
tests/probes/xcd_probe.hip (which XCD runs each workgroup, from the XCC_ID register).

The chunk kernels' schedules put the two workgroups that read the same inputs a multiple of
8 workgroup indices apart: the two value-column halves of a chain are 8 items apart
(split_item in csrc/kda_mfma.h and the work lists of chunk_plan_kernel), a later segment's
zero-state and transition items H apart (H a multiple of 8 for that to hold). On a device
that dispatches workgroups round-robin over its 8 XCDs both then run on one XCD and the
second reads the inputs through the first's L2. Results do not depend on it; the measured
HBM traffic does."""

import ctypes
import os

import numpy as np
import pytest

LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "probes", "libxcd_probe.so")


def _probe():
    lib = ctypes.CDLL(LIB)
    lib.xcd_of_workgroups.argtypes = [ctypes.POINTER(ctypes.c_int), ctypes.c_int, ctypes.c_int]
    lib.xcd_of_workgroups.restype = ctypes.c_int
    return lib


def test_probe_library_exports_its_entry_point():
    assert os.path.exists(LIB), "tests/probes is not built; run __graft_entry__.build()"
    assert _probe().xcd_of_workgroups is not None


@pytest.mark.gpu
@pytest.mark.parametrize("threads", [64, 512])
def test_workgroups_eight_apart_share_an_xcd(threads):
    """4096 workgroups of 64 or 512 threads (512: the chunk kernels' workgroup size): they
    run on 8 XCDs, and workgroups i and i + 8 always on the same one."""
    n = 4096
    out = (ctypes.c_int * n)()
    assert _probe().xcd_of_workgroups(out, n, threads) == 0
    xcd = np.frombuffer(out, dtype=np.int32).copy()
    assert sorted(set(xcd.tolist())) == list(range(8)), f"XCDs seen: {sorted(set(xcd.tolist()))}"
    assert np.array_equal(xcd[8:], xcd[:-8]), "workgroups 8 apart ran on different XCDs"
