"""GPU parity with infinities and NaN in the inputs.

The kernels pad a batch of points to whole request rounds with slots that
hold no point: those read zero rows with weight zero, so they add +0 whatever
the table holds.  These tests put +-Inf into the feature rows of the last
(and first) point of every interval, an Inf weight on one point, and a zero
weight on an Inf row (0 * Inf = NaN), at interval lengths around the round
and batch sizes of each row geometry and past the one-wave and channel-split
limits.  The oracle's fp64 sums give the expected NaN / +Inf / -Inf pattern
(IEEE arithmetic decides it, whatever the summation order); every other
element must match the oracle to the usual scaled tolerance.

OCP e4m3 has no infinities: its rows carry the NaN codes instead (0x7F where
the other types hold +Inf, 0xFF where they hold -Inf), so an e4m3 interval's
first or last point reaches its cell as NaN, and an Inf weight turns every
finite channel of its point into +Inf.
"""
import numpy as np
import pytest
import torch

import depth_weighted_scatter_amd as dws
import oracle
from gpu_util import TOL, dev, say, scaled_error, to_gpu

pytestmark = pytest.mark.gpu

LENGTHS = [1, 2, 5, 6, 7, 11, 12, 13, 16, 17, 18, 19, 23, 24, 25, 36, 47, 48, 49, 53, 54, 55,
           60, 63, 64, 65, 72, 95, 96, 97, 150, 300, 385, 700]


@pytest.fixture(scope="module", autouse=True)
def _setup():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    oracle.build(force=False)
    dws._load()


def _inputs(C, np_dtype, seed):
    """Rows with values in [0.5, 1.5) (no cancellation), one row per point,
    +Inf in one channel of the last point's row of every interval, -Inf in
    another channel of the first point's row of every third interval, and
    weights in [0.25, 1) with one Inf weight (the length-5 interval: +Inf in
    every channel) and one zero weight on an Inf row (the length-17 interval:
    0 * Inf = NaN in that channel)."""
    rng = np.random.default_rng(seed)
    lens = np.array(LENGTHS)
    starts = np.r_[0, np.cumsum(lens)[:-1]]
    N = int(lens.sum())
    rows = (0.5 + rng.random((N, C))).astype(np_dtype)
    w = (0.25 + 0.75 * rng.random(N)).astype(np_dtype)
    for i, (s0, n) in enumerate(zip(starts, lens)):
        rows[s0 + n - 1, (7 * i) % C] = np.inf
        if i % 3 == 0:
            rows[s0, (7 * i + 1) % C] = -np.inf
    five, seventeen = LENGTHS.index(5), LENGTHS.index(17)
    w[starts[five] + 2] = np.inf
    w[starts[seventeen] + lens[seventeen] - 1] = 0
    return lens, starts, rows, w


def _rows_of(dtype, rows):
    """Rows in the feature type: fp16 / fp32 as they are; e4m3 as codes, with
    the infinities replaced by the format's NaN codes."""
    if dtype != "e4m3":
        return rows
    finite = np.where(np.isfinite(rows), rows, 1.0).astype(np.float32)
    codes = torch.from_numpy(finite).to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
    codes[np.isposinf(rows)] = 0x7F
    codes[np.isneginf(rows)] = 0xFF
    return codes


def _check(got, ref, ref_abs, dtype, label):
    for name, f in (("NaN", np.isnan), ("+Inf", np.isposinf), ("-Inf", np.isneginf)):
        a, b = f(got), f(ref)
        assert np.array_equal(a, b), (f"{label}: {name} pattern differs at "
                                      f"{np.argwhere(a != b)[:5].tolist()}")
    fin = np.isfinite(ref)
    assert fin.sum() > 0.9 * fin.size
    e = scaled_error(np.where(fin, got, 0), np.where(fin, ref, 0), np.where(fin, ref_abs, 0))
    say(f"  {label}: non-finite {int((~fin).sum())} elements match, finite scaled err {e:.2e}")
    assert e <= TOL[dtype], f"{label}: scaled error {e}"


# (feature dtype, C): ten-chunk rows (6 points per instruction), 16-chunk
# rows, five-chunk rows, fp32 16-chunk rows, 32-chunk rows, e4m3 rows of ten
# 8-byte chunks and of sixteen 16-byte chunks (split by channels in segment
# reductions)
GEOMETRIES = [("f16", 80), ("f16", 128), ("f16", 40), ("f32", 64), ("f16", 256),
              ("e4m3", 80), ("e4m3", 256)]


@pytest.mark.parametrize("dtype,C", GEOMETRIES, ids=[f"{a}-C{b}" for a, b in GEOMETRIES])
def test_forward_nonfinite_rows_and_weights(dtype, C):
    np_dtype = np.float32 if dtype == "f32" else np.float16
    lens, starts, rows, w = _inputs(C, np_dtype, 70 + C)
    rows = _rows_of(dtype, rows)
    n_iv = lens.size
    say(f"[nonfinite forward {dtype} C={C}] intervals={n_iv} N={rows.shape[0]}")
    # one cell per interval, every other cell empty
    cells = 2 * np.arange(n_iv, dtype=np.int32)
    n_cells = 2 * n_iv + 1
    m = {"ranks_depth": np.arange(rows.shape[0], dtype=np.int32),
         "ranks_feat": np.arange(rows.shape[0], dtype=np.int32),
         "ranks_bev": np.repeat(cells, lens).astype(np.int32),
         "interval_starts": starts.astype(np.int32), "interval_lengths": lens.astype(np.int32)}
    ref, ref_abs = oracle.forward(w, rows, dtype, 1.0, C, m, n_cells, with_abs=True)
    gm = dws.BevMap(*(to_gpu(m[k]) for k in ("ranks_depth", "ranks_feat", "ranks_bev",
                                             "interval_starts", "interval_lengths")),
                    n_points=int(lens.sum()), n_intervals=n_iv)
    out = torch.full((n_cells, C), 7.0, dtype=torch.float32, device=dev())
    dws.bevpool_forward(to_gpu(w), to_gpu(rows), gm, n_cells, out=out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert (got[1::2] == 0).all(), "empty cells not zero"
    _check(got, ref, ref_abs, dtype, f"forward {dtype} C={C}")


@pytest.mark.parametrize("dtype,C", GEOMETRIES, ids=[f"{a}-C{b}" for a, b in GEOMETRIES])
def test_segment_reduce_nonfinite_rows_and_weights(dtype, C):
    np_dtype = np.float32 if dtype == "f32" else np.float16
    lens, starts, rows, w = _inputs(C, np_dtype, 90 + C)
    rows = _rows_of(dtype, rows)
    say(f"[nonfinite segments {dtype} C={C}] segments={lens.size} N={rows.shape[0]}")
    off = np.r_[starts, lens.sum()].astype(np.int32)
    idx = np.arange(rows.shape[0], dtype=np.int32)
    ref, ref_abs = oracle.segment_reduce(w, rows, dtype, 1.0, idx, off, with_abs=True)
    out = torch.full((lens.size, C), 7.0, dtype=torch.float32, device=dev())
    dws.bevpool_segment_reduce(to_gpu(w), to_gpu(rows), to_gpu(idx), to_gpu(off), out=out)
    torch.cuda.synchronize()
    _check(out.cpu().numpy(), ref, ref_abs, dtype, f"segments {dtype} C={C}")
