"""Helpers shared by the GPU parity tests: move seeded numpy inputs to the
GPU, call the library through its C ABI binding, and compare with the CPU
oracle.  Nothing here computes any part of BEV pooling itself."""
from __future__ import annotations

import sys

import numpy as np
import torch

import depth_weighted_scatter_amd as dws
import oracle

MAP_KEYS = ("ranks_depth", "ranks_feat", "ranks_bev", "interval_starts", "interval_lengths")

# Tolerances on the error scaled by sum |d * f| over the cell's terms: fp32
# accumulation of n terms is within about n * 2^-24 of that scale (n <= 1440
# here, i.e. <= 1e-4); 1e-3 and 2e-2 are the stated acceptance bars.
TOL = {"f32": 1e-3, "f16": 1e-3, "e4m3": 2e-2}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev():
    return torch.device("cuda:0")


def to_gpu(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def gpu_map(point_cell: np.ndarray, n_img, D, H, W, n_cells, capacity=None) -> dws.BevMap:
    m = dws.bevpool_build_map(to_gpu(point_cell.astype(np.int32)), n_img, D, H, W, n_cells,
                              capacity=capacity)
    torch.cuda.synchronize()
    return m


def map_to_numpy(m: dws.BevMap) -> dict:
    d = {k: getattr(m, k).cpu().numpy() for k in MAP_KEYS}
    d["n_points"], d["n_intervals"] = m.n_points, m.n_intervals
    return d


def assert_maps_equal(got: dict, ref: dict, label=""):
    assert got["n_points"] == ref["n_points"], f"{label}: n_points {got['n_points']} != {ref['n_points']}"
    assert got["n_intervals"] == ref["n_intervals"], f"{label}: n_intervals differ"
    for k in MAP_KEYS:
        a, b = got[k], ref[k]
        if not np.array_equal(a, b):
            bad = np.nonzero(a != b)[0] if a.shape == b.shape else []
            raise AssertionError(f"{label}: {k} differs (first at {bad[:5]})")


def map_from_numpy(ref: dict) -> dws.BevMap:
    t = {k: to_gpu(ref[k].astype(np.int32)) for k in MAP_KEYS}
    return dws.BevMap(**t, n_points=ref["n_points"], n_intervals=ref["n_intervals"])


def feat_tensor(feat: np.ndarray) -> torch.Tensor:
    return to_gpu(feat)          # uint8 e4m3 codes are passed as uint8


def gpu_forward(depth, feat, feat_scale, m: dws.BevMap, n_cells, C) -> np.ndarray:
    out = torch.full((n_cells, C), float("nan"), dtype=torch.float32, device=dev())
    dws.bevpool_forward(to_gpu(depth), feat_tensor(feat), m, n_cells, feat_scale=feat_scale, out=out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def scaled_error(got: np.ndarray, ref: np.ndarray, ref_abs: np.ndarray) -> float:
    """max |got - ref| / sum|terms|, with 0/0 taken as 0 (and x/0 as inf)."""
    err = np.abs(got.astype(np.float64) - ref)
    with np.errstate(divide="ignore", invalid="ignore"):
        e = np.where(ref_abs > 0, err / ref_abs, np.where(err > 0, np.inf, 0.0))
    return float(e.max()) if e.size else 0.0


def check_forward(got, ref, ref_abs, feat_dtype, occupied_cells, label=""):
    assert np.isfinite(got).all(), f"{label}: non-finite output (unwritten element?)"
    e = scaled_error(got, ref, ref_abs)
    normwise = float(np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-300)) if ref.size else 0.0
    say(f"  {label}: scaled err {e:.3e}, normwise {normwise:.3e}, "
        f"max abs {float(np.abs(got - ref).max()) if ref.size else 0.0:.3e}")
    assert e <= TOL[feat_dtype], f"{label}: scaled error {e} > {TOL[feat_dtype]}"
    empty = np.ones(got.shape[0], bool)
    empty[occupied_cells] = False
    assert (got[empty] == 0).all(), f"{label}: empty cells not exactly zero"
    return e


def oracle_reference(depth, feat, feat_dtype, feat_scale, C, ref_map, n_cells):
    return oracle.forward(depth, feat, feat_dtype, feat_scale, C, ref_map, n_cells, with_abs=True)
