"""bevpool_build_map_no_alloc (the map build on the library's static device
workspace) against bevpool_build_map (caller workspace), through the C ABI.

Both must give the same five arrays and counts bit for bit, on two calls in
a row with the second smaller than the first (the static workspace keeps
the first call's contents), after an error return, and on a repeat of the
first call.  Each map is also checked against the oracle's.
"""
import ctypes

import numpy as np
import pytest
import torch

import depth_weighted_scatter_amd as dws
import oracle
import workloads as W
from gpu_util import MAP_KEYS, assert_maps_equal, gpu_map, map_to_numpy, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _setup():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    oracle.build(force=False)
    dws._load()


def _no_alloc(pc: np.ndarray, n_img, D, H, Wd, n_cells, capacity=None):
    """Calls the C entry point directly; returns (status, map dict)."""
    lib = dws._load()
    dev = torch.device("cuda:0")
    P = n_img * D * H * Wd
    cap = P if capacity is None else capacity
    pc_d = torch.from_numpy(pc.astype(np.int32)).to(dev)
    arrs = [torch.full((max(cap, 1),), -7, dtype=torch.int32, device=dev) for _ in range(5)]
    n_pts, n_iv = ctypes.c_int32(), ctypes.c_int32()
    torch.cuda.synchronize()
    rc = lib.bevpool_build_map_no_alloc(pc_d.data_ptr(), n_img, D, H, Wd, n_cells,
                                        *(a.data_ptr() for a in arrs), cap,
                                        ctypes.byref(n_pts), ctypes.byref(n_iv),
                                        torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    N, I = n_pts.value, n_iv.value
    got = {k: a[:(N if k.startswith("ranks") else I)].cpu().numpy() for k, a in zip(MAP_KEYS, arrs)}
    got["n_points"], got["n_intervals"] = N, I
    return rc, got


def _case(k):
    wl = W.make_workload(k)
    s = wl.spec
    return wl.point_cell, (s.n_img, s.D, s.H, s.W, s.n_cells)


def test_no_alloc_matches_workspace_build_twice_then_smaller():
    big = _case(3)                 # 2.0 M-point frustum: 39 MiB of the 80 MiB workspace
    small = _case(1)               # 249 K points
    tiny = _case(0)                # 256 points
    for label, (pc, geo) in [("hires (first call)", big), ("bevdet (smaller)", small),
                             ("tiny (smaller again)", tiny), ("hires (again)", big)]:
        say(f"[no-alloc map build] {label}: P={pc.size}")
        rc, got = _no_alloc(pc, *geo)
        assert rc == 0, f"{label}: status {rc}"
        ref = map_to_numpy(gpu_map(pc, *geo))            # caller-workspace entry point
        assert_maps_equal(got, ref, f"{label} vs bevpool_build_map")
        assert_maps_equal(got, oracle.build_map(pc, *geo), f"{label} vs oracle")


def test_no_alloc_after_errors():
    """A bad cell or a too-small capacity returns its status; the next call
    (smaller) is still exact: the build clears its counters itself."""
    pc, geo = _case(1)
    bad = pc.copy()
    bad[12345] = geo[-1] + 5                  # a cell past the grid
    say("[no-alloc map build] bad cell, then capacity, then a smaller valid call")
    rc, _ = _no_alloc(bad, *geo)
    assert rc == -6
    rc, got = _no_alloc(pc, *geo, capacity=1000)
    assert rc == -5 and got["n_points"] == int((pc >= 0).sum())
    pc0, geo0 = _case(0)
    rc, got = _no_alloc(pc0, *geo0)
    assert rc == 0
    assert_maps_equal(got, oracle.build_map(pc0, *geo0), "after errors")


def test_no_alloc_binding_matches():
    """The Python binding of the same name, with caller-provided arrays."""
    pc, geo = _case(2)
    dev = torch.device("cuda:0")
    arrays = [torch.empty(pc.size, dtype=torch.int32, device=dev) for _ in range(5)]
    say("[no-alloc map build] binding")
    m = dws.bevpool_build_map_no_alloc(torch.from_numpy(pc).to(dev), *geo, arrays=arrays)
    torch.cuda.synchronize()
    assert_maps_equal(map_to_numpy(m), oracle.build_map(pc, *geo), "binding")
