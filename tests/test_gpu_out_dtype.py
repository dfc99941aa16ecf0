"""GPU parity of bevpool_forward_ex: fp32 accumulation with the output rounded
once, to nearest-even, to float16 or bfloat16 at the store.

Bound used against the oracle's fp64 sum s with term scale A = sum |d * f|:
the kernel's fp32 sum s' is within TOL * A of s (the accumulation bar of the
fp32-output tests), and rounding s' to the output type moves it by at most
u * |s'| (u = 2^-11 for binary16, 2^-8 for bfloat16) plus half the smallest
subnormal step, so |out - s| <= TOL*A + u*(|s| + TOL*A) + tiny.
"""
import functools

import numpy as np
import pytest
import torch

import depth_weighted_scatter_amd as dws
import oracle
import workloads as W
from gpu_util import TOL, dev, feat_tensor, gpu_map, map_from_numpy, oracle_reference, say, to_gpu

pytestmark = pytest.mark.gpu

UNIT = {torch.float16: 2.0 ** -11, torch.bfloat16: 2.0 ** -8}
TINY = {torch.float16: 2.0 ** -25, torch.bfloat16: 2.0 ** -134}
OUT_DTYPES = [torch.float16, torch.bfloat16]


@pytest.fixture(scope="module", autouse=True)
def _setup():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    oracle.build(force=False)
    dws._load()


def _forward_ex(depth, feat, scale, m, n_cells, C, out_dtype) -> torch.Tensor:
    out = torch.full((n_cells, C), float("nan"), dtype=out_dtype, device=dev())
    dws.bevpool_forward_ex(to_gpu(depth), feat_tensor(feat), m, n_cells, out_dtype=out_dtype,
                           feat_scale=scale, out=out)
    torch.cuda.synchronize()
    return out.cpu()


def _forward_f32(depth, feat, scale, m, n_cells, C) -> torch.Tensor:
    out = dws.bevpool_forward(to_gpu(depth), feat_tensor(feat), m, n_cells, feat_scale=scale)
    torch.cuda.synchronize()
    return out.cpu()


def _check_narrow(got: torch.Tensor, ref, ref_abs, feat_dtype, occupied, label):
    out_dtype = got.dtype
    g = got.to(torch.float64).numpy()
    assert np.isfinite(g).all(), f"{label}: non-finite output (unwritten element?)"
    tol = TOL[feat_dtype]
    bound = tol * ref_abs + UNIT[out_dtype] * (np.abs(ref) + tol * ref_abs) + TINY[out_dtype]
    err = np.abs(g - ref)
    worst = float((err / bound).max()) if err.size else 0.0
    say(f"  {label}: max err/bound {worst:.3f}")
    assert (err <= bound).all(), f"{label}: error beyond bound (ratio {worst})"
    empty = np.ones(g.shape[0], bool)
    empty[occupied] = False
    assert (got[torch.from_numpy(empty)].view(torch.int16) == 0).all(), f"{label}: empty cells"


@functools.lru_cache(maxsize=2)
def _workload_reference(k):
    wl = W.make_workload(k)
    s = wl.spec
    ref = oracle.build_map(wl.point_cell, s.n_img, s.D, s.H, s.W, s.n_cells)
    out_ref, out_abs = oracle_reference(wl.depth, wl.feat, s.feat_dtype, wl.feat_scale, s.C, ref,
                                        s.n_cells)
    return wl, ref, out_ref, out_abs


@pytest.mark.parametrize("out_dtype", OUT_DTYPES, ids=["f16", "bf16"])
@pytest.mark.parametrize("k", [0, 1, 2, 4, 9])
def test_forward_ex_narrow_output_on_workloads(out_dtype, k):
    wl, ref, out_ref, out_abs = _workload_reference(k)
    s = wl.spec
    say(f"[forward_ex workload {k} {s.name} -> {out_dtype}]")
    m = gpu_map(wl.point_cell, s.n_img, s.D, s.H, s.W, s.n_cells)
    got = _forward_ex(wl.depth, wl.feat, wl.feat_scale, m, s.n_cells, s.C, out_dtype)
    _check_narrow(got, out_ref, out_abs, s.feat_dtype, ref["ranks_bev"], f"workload {k}")
    # The fp32 sums are those of bevpool_forward; only the final rounding
    # differs, and it must be round-to-nearest-even of exactly those sums.
    f32 = _forward_f32(wl.depth, wl.feat, wl.feat_scale, m, s.n_cells, s.C)
    assert torch.equal(got.view(torch.int16), f32.to(out_dtype).view(torch.int16))


@pytest.mark.parametrize("k", [1, 2])
def test_forward_ex_f32_output_is_bevpool_forward(k):
    wl = W.make_workload(k)
    s = wl.spec
    say(f"[forward_ex workload {k} f32 output]")
    m = gpu_map(wl.point_cell, s.n_img, s.D, s.H, s.W, s.n_cells)
    got = _forward_ex(wl.depth, wl.feat, wl.feat_scale, m, s.n_cells, s.C, torch.float32)
    f32 = _forward_f32(wl.depth, wl.feat, wl.feat_scale, m, s.n_cells, s.C)
    assert torch.equal(got.view(torch.int32), f32.view(torch.int32))


CHANNEL_CASES = [("f32", 4), ("f32", 12), ("f16", 8), ("f16", 80), ("f16", 512),
                 ("e4m3", 8), ("e4m3", 40), ("e4m3", 528)]


@pytest.mark.parametrize("out_dtype", OUT_DTYPES, ids=["f16", "bf16"])
@pytest.mark.parametrize("feat_dtype,C", CHANNEL_CASES,
                         ids=[f"{a}-C{b}" for a, b in CHANNEL_CASES])
def test_forward_ex_channel_widths(feat_dtype, C, out_dtype):
    """Rows of 1 to 128 output quads, ragged against the 64-lane wave, with
    empty cells between, before and after the occupied ones."""
    rng = np.random.default_rng(C * 3 + len(feat_dtype))
    n_img, D, H, Wd, n_cells = 2, 5, 4, 29, 83
    P = n_img * D * H * Wd
    pc = W.make_random_cells(rng, P, n_cells, p_drop=0.4, hot_cells=1)
    pc[pc == 0] = -1
    pc[pc == n_cells - 1] = -1
    depth = rng.random((n_img, D, H, Wd))
    feat = rng.standard_normal((n_img, H, Wd, C))
    scale = 1.0
    if feat_dtype == "f32":
        depth, feat = depth.astype(np.float32), feat.astype(np.float32)
    elif feat_dtype == "f16":
        depth, feat = depth.astype(np.float16), feat.astype(np.float16)
    else:
        feat, scale = W.quantize_e4m3(feat.astype(np.float16))
        depth = depth.astype(np.float16)
    say(f"[forward_ex C={C} {feat_dtype} -> {out_dtype}]")
    ref = oracle.build_map(pc, n_img, D, H, Wd, n_cells)
    out_ref, out_abs = oracle_reference(depth, feat, feat_dtype, scale, C, ref, n_cells)
    got = _forward_ex(depth, feat, scale, map_from_numpy(ref), n_cells, C, out_dtype)
    _check_narrow(got, out_ref, out_abs, feat_dtype, ref["ranks_bev"], f"C={C}")


@pytest.mark.parametrize("out_dtype", OUT_DTYPES, ids=["f16", "bf16"])
def test_forward_ex_length_one_bit_exact(out_dtype):
    """One point per cell: the fp32 product d * f of two fp16 values is
    exact, so the output must be the oracle's value rounded once to the
    output type (numpy / torch round-to-nearest-even on the CPU)."""
    rng = np.random.default_rng(23)
    n_img, D, H, Wd, C = 1, 4, 8, 16, 80
    P = n_img * D * H * Wd
    n_cells = P + 9
    pc = rng.permutation(n_cells)[:P].astype(np.int32)
    pc[rng.random(P) < 0.2] = -1
    depth = rng.random((n_img, D, H, Wd)).astype(np.float16)
    feat = (rng.standard_normal((n_img, H, Wd, C)) * 3).astype(np.float16)
    say(f"[forward_ex length-1 -> {out_dtype}]")
    ref = oracle.build_map(pc, n_img, D, H, Wd, n_cells)
    out_ref = oracle.forward(depth, feat, "f16", 1.0, C, ref, n_cells)
    exact32 = torch.from_numpy(out_ref.astype(np.float32))
    assert np.array_equal(exact32.numpy().astype(np.float64), out_ref)
    got = _forward_ex(depth, feat, 1.0, map_from_numpy(ref), n_cells, C, out_dtype)
    assert torch.equal(got.view(torch.int16), exact32.to(out_dtype).view(torch.int16))


def test_forward_ex_f16_overflow_and_bf16_range():
    """Sums beyond binary16's range round to +-inf in an fp16 output and stay
    finite in bfloat16, as nearest-even rounding of the fp32 sum gives."""
    n_img, D, H, Wd, C = 1, 1, 4, 4, 8
    P = 16
    pc = np.arange(P, dtype=np.int32)
    depth = np.ones((n_img, D, H, Wd), np.float32)
    feat = np.zeros((n_img, H, Wd, C), np.float32)
    vals = np.array([65504.0, 65519.0, 65520.0, -70000.0, 1e6, 3.0e38, -1e-30, 6e-8],
                    np.float32)
    feat.reshape(P, C)[:, :] = vals[None, :]
    say("[forward_ex fp16 overflow]")
    ref = oracle.build_map(pc, n_img, D, H, Wd, P)
    m = map_from_numpy(ref)
    out_ref = oracle.forward(depth, feat, "f32", 1.0, C, ref, P)
    for out_dtype in OUT_DTYPES:
        got = _forward_ex(depth, feat, 1.0, m, P, C, out_dtype)
        want = torch.from_numpy(out_ref.astype(np.float32)).to(out_dtype)
        assert torch.equal(got.view(torch.int16), want.view(torch.int16)), out_dtype
    got16 = _forward_ex(depth, feat, 1.0, m, P, C, torch.float16)[0]
    assert got16[0] == 65504 and got16[1] == 65504 and torch.isinf(got16[2:5]).all()


@pytest.mark.parametrize("out_dtype", OUT_DTYPES, ids=["f16", "bf16"])
def test_forward_ex_no_points_zero_fills(out_dtype):
    n_cells, C = 1237, 80
    out = torch.full((n_cells, C), float("nan"), dtype=out_dtype, device=dev())
    empty = dws.BevMap(*(torch.zeros(1, dtype=torch.int32, device=dev()) for _ in range(5)),
                       n_points=0, n_intervals=0)
    feat = torch.zeros((4, C), dtype=torch.float16, device=dev())
    depth = torch.zeros(4, dtype=torch.float16, device=dev())
    dws.bevpool_forward_ex(depth, feat, empty, n_cells, out_dtype=out_dtype, out=out)
    torch.cuda.synchronize()
    assert (out.view(torch.int16) == 0).all()


def test_forward_ex_long_intervals_narrow():
    """Intervals past the one-wave limit go through the block role; its
    rounded store and gap zeroing must match the fp32 path's sums."""
    rng = np.random.default_rng(31)
    n_img, D, H, Wd, C, n_cells = 1, 8, 16, 40, 80, 300
    P = n_img * D * H * Wd
    pc = W.make_random_cells(rng, P, n_cells, p_drop=0.5)
    pc[::3] = 150
    pc[1::7] = 299
    depth = rng.random((n_img, D, H, Wd)).astype(np.float16)
    feat = rng.standard_normal((n_img, H, Wd, C)).astype(np.float16)
    ref = oracle.build_map(pc, n_img, D, H, Wd, n_cells)
    assert ref["interval_lengths"].max() > 96
    m = map_from_numpy(ref)
    out_ref, out_abs = oracle_reference(depth, feat, "f16", 1.0, C, ref, n_cells)
    f32 = _forward_f32(depth, feat, 1.0, m, n_cells, C)
    for out_dtype in OUT_DTYPES:
        say(f"[forward_ex long intervals -> {out_dtype}]")
        got = _forward_ex(depth, feat, 1.0, m, n_cells, C, out_dtype)
        _check_narrow(got, out_ref, out_abs, "f16", ref["ranks_bev"], "long")
        assert torch.equal(got.view(torch.int16), f32.to(out_dtype).view(torch.int16))
