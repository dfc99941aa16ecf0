"""The C ABI used from plain C: tests/c_abi/bevpool_example.c compiles as C99
against include/bevpool.h (CPU), and on the GPU it builds the map and pools a
problem written here; its results are checked against the CPU oracle like the
Python-driven parity tests (map bit-exact, output within the scaled bound)."""
import os
import subprocess

import numpy as np
import pytest

import oracle
import workloads as W

HERE = os.path.dirname(os.path.abspath(__file__))
C_ABI = os.path.join(HERE, "c_abi")

TOL = {"f32": 1e-3, "f16": 1e-3, "e4m3": 2e-2}
CODE = {"f32": 0, "f16": 1, "e4m3": 2, "bf16": 3}
UNIT = {"f32": 0.0, "f16": 2.0 ** -11, "bf16": 2.0 ** -8}
TINY = {"f32": 0.0, "f16": 2.0 ** -25, "bf16": 2.0 ** -134}


def _builder():
    import importlib.util
    spec = importlib.util.spec_from_file_location("build_example",
                                                  os.path.join(C_ABI, "build_example.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_c_example_compiles_as_c99(tmp_path):
    lib = os.path.join(os.path.dirname(HERE), "depth_weighted_scatter_amd", "libbevpool.so")
    if not os.path.exists(lib):
        pytest.skip("libbevpool.so is not built")
    out = _builder().build(str(tmp_path / "bevpool_example"), werror=True)
    assert os.path.exists(out)


def _problem(case):
    if case == "tiny_f32":
        wl = W.make_workload(0)
        s = wl.spec
        return (wl.point_cell, wl.depth, wl.feat, s.n_img, s.D, s.H, s.W, s.n_cells, s.C, "f32",
                "f32", "f32")
    rng = np.random.default_rng(17)
    n_img, D, H, Wd, n_cells = 2, 6, 5, 37, 97
    P = n_img * D * H * Wd
    pc = W.make_random_cells(rng, P, n_cells, p_drop=0.3, hot_cells=2)
    depth = rng.random((n_img, D, H, Wd)).astype(np.float16)
    if case == "f16_c80_out_f16":
        feat = rng.standard_normal((n_img, H, Wd, 80)).astype(np.float16)
        return pc, depth, feat, n_img, D, H, Wd, n_cells, 80, "f16", "f16", "f16"
    q, _ = W.quantize_e4m3(rng.standard_normal((n_img, H, Wd, 40)).astype(np.float16))
    return pc, depth, q, n_img, D, H, Wd, n_cells, 40, "e4m3", "f16", "bf16"


@pytest.mark.gpu
@pytest.mark.parametrize("case", ["tiny_f32", "f16_c80_out_f16", "e4m3_c40_out_bf16"])
def test_c_example_on_gpu(case, tmp_path):
    exe = os.path.join(C_ABI, "bevpool_example")
    if not os.path.exists(exe):
        _builder().build(exe)
    pc, depth, feat, n_img, D, H, Wd, n_cells, C, fdt, ddt, odt = _problem(case)
    d = tmp_path
    (d / "meta.txt").write_text(f"{n_img} {D} {H} {Wd} {n_cells} {C} {CODE[fdt]} {CODE[ddt]} "
                                f"{CODE[odt]}\n")
    np.ascontiguousarray(pc, np.int32).tofile(d / "point_cell")
    np.ascontiguousarray(depth).tofile(d / "depth")
    np.ascontiguousarray(feat).tofile(d / "feat")
    print(f"[C example {case}]", flush=True)
    r = subprocess.run([exe, str(d)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, f"C example failed ({r.returncode}): {r.stdout}{r.stderr}"

    ref = oracle.build_map(pc, n_img, D, H, Wd, n_cells)
    raw = np.fromfile(d / "map", np.int32)
    N, I = int(raw[0]), int(raw[1])
    assert (N, I) == (ref["n_points"], ref["n_intervals"])
    parts = np.split(raw[2:], np.cumsum([N, N, N, I])[:4])
    for k, got in zip(("ranks_depth", "ranks_feat", "ranks_bev", "interval_starts",
                       "interval_lengths"), parts):
        assert np.array_equal(got, ref[k]), k

    if odt == "f32":
        out = np.fromfile(d / "out", np.float32)
    elif odt == "f16":
        out = np.fromfile(d / "out", np.float16).astype(np.float32)
    else:
        out = (np.fromfile(d / "out", np.uint16).astype(np.uint32) << 16).view(np.float32)
    out = out.reshape(n_cells, C).astype(np.float64)
    # the C example passes feat_scale = 1.0 (e4m3 codes are read unscaled)
    ref_out, ref_abs = oracle.forward(depth, feat, fdt, 1.0, C, ref, n_cells, with_abs=True)
    tol = TOL[fdt]
    bound = tol * ref_abs + UNIT[odt] * (np.abs(ref_out) + tol * ref_abs) + TINY[odt]
    assert np.isfinite(out).all()
    assert (np.abs(out - ref_out) <= bound).all()
    empty = np.setdiff1d(np.arange(n_cells), ref["ranks_bev"])
    assert (out[empty] == 0).all()

