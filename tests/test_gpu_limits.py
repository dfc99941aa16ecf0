"""GPU parity at the size limits of the C ABI.

* Feature tables at the byte limit of the C ABI (2^32 - 4096 bytes, and
  under 2^31 elements), with the gathered rows at the top of the table, so
  the kernel's 32-bit unsigned row offsets run up to their largest values.
* An output of n_cells*C just under 2^31 elements (8.6 GB of fp32), with an
  occupied cell every 64 cells plus the first and the last cell, so every
  element is written (checked against a NaN fill) and the empty ones are 0.

The oracle works on the same points with the occupied cells renumbered
densely and only the gathered rows kept: renaming cells and rows changes no
sum, and it keeps the host-side arrays small.
"""
import numpy as np
import pytest
import torch

import depth_weighted_scatter_amd as dws
import oracle
import workloads as W
from gpu_util import check_forward, dev, map_to_numpy, say, to_gpu

pytestmark = pytest.mark.gpu

INT32_MAX = 2 ** 31 - 1


@pytest.fixture(scope="module", autouse=True)
def _setup():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    oracle.build(force=False)
    dws._load()


def _map_from_cells(cells: np.ndarray, ranks_depth: np.ndarray, ranks_feat: np.ndarray) -> dict:
    """Five-array map for points already ordered by cell (non-decreasing)."""
    N = cells.size
    starts = np.flatnonzero(np.r_[True, cells[1:] != cells[:-1]]).astype(np.int32)
    lengths = np.diff(np.r_[starts, N]).astype(np.int32)
    return {"ranks_depth": ranks_depth.astype(np.int32), "ranks_feat": ranks_feat.astype(np.int32),
            "ranks_bev": cells.astype(np.int32), "interval_starts": starts,
            "interval_lengths": lengths, "n_points": N, "n_intervals": starts.size}


def _gpu_map(m: dict) -> dws.BevMap:
    return dws.BevMap(*(to_gpu(m[k]) for k in ("ranks_depth", "ranks_feat", "ranks_bev",
                                                 "interval_starts", "interval_lengths")),
                      n_points=m["n_points"], n_intervals=m["n_intervals"])


LARGE_TABLES = [("f16", 80), ("f32", 64), ("e4m3", 512)]


@pytest.mark.parametrize("feat_dtype,C", LARGE_TABLES, ids=[f"{a}-C{b}" for a, b in LARGE_TABLES])
def test_forward_largest_feature_table(feat_dtype, C):
    eb = {"f32": 4, "f16": 2, "e4m3": 1}[feat_dtype]
    n_rows = min(INT32_MAX // C, dws.MAX_TABLE_BYTES // (C * eb))
    say(f"[largest table {feat_dtype} C={C}] rows={n_rows} bytes={n_rows * C * eb}")
    rng = np.random.default_rng(41)
    # rows used: the top 200 of the table and 100 elsewhere
    used = np.unique(np.r_[np.arange(n_rows - 200, n_rows), rng.integers(0, n_rows, 100)])
    vals = rng.standard_normal((used.size, C))
    scale = 1.0
    if feat_dtype == "f32":
        vals, tdt, ddt = vals.astype(np.float32), torch.float32, np.float32
    elif feat_dtype == "f16":
        vals, tdt, ddt = vals.astype(np.float16), torch.float16, np.float16
    else:
        vals, scale = W.quantize_e4m3(vals.astype(np.float16))
        tdt, ddt = torch.uint8, np.float16
    # points: 40 cells, lengths 1..300 (some past the one-wave limit)
    n_cells = 40
    lengths = np.r_[rng.integers(1, 40, 35), [97, 150, 300, 1, 200]]
    cells = np.repeat(np.sort(rng.choice(n_cells + 20, n_cells, replace=False)), lengths)
    n_cells += 20
    N = cells.size
    pick = rng.integers(0, used.size, N)
    n_depth = 5000
    depth = rng.random(n_depth).astype(ddt)
    ranks_depth = rng.integers(0, n_depth, N)
    m_gpu = _map_from_cells(cells, ranks_depth, used[pick])
    m_ref = _map_from_cells(cells, ranks_depth, pick)          # rows renumbered densely

    feat = torch.zeros((n_rows, C), dtype=tdt, device=dev())
    feat[torch.from_numpy(used).to(dev())] = torch.from_numpy(vals).to(dev())
    out = torch.full((n_cells, C), float("nan"), dtype=torch.float32, device=dev())
    dws.bevpool_forward(to_gpu(depth), feat, _gpu_map(m_gpu), n_cells, feat_scale=scale, out=out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    del feat
    torch.cuda.empty_cache()
    ref, ref_abs = oracle.forward(depth, vals, feat_dtype, scale, C, m_ref, n_cells, with_abs=True)
    check_forward(got, ref, ref_abs, feat_dtype, m_ref["ranks_bev"], f"table {feat_dtype}")


def test_forward_largest_output():
    C = 8
    n_cells = INT32_MAX // C                                    # 268,435,455 cells, 8.6 GB fp32
    rng = np.random.default_rng(43)
    occ = np.r_[0, np.arange(64, n_cells - 1, 64), n_cells - 1].astype(np.int64)
    lengths = rng.integers(1, 4, occ.size)
    cells = np.repeat(occ, lengths)
    N = cells.size
    n_rows, n_depth = 10000, 4096
    feat = rng.standard_normal((n_rows, C)).astype(np.float16)
    depth = rng.random(n_depth).astype(np.float16)
    ranks_depth = rng.integers(0, n_depth, N)
    ranks_feat = rng.integers(0, n_rows, N)
    say(f"[largest output] n_cells={n_cells} occupied={occ.size} points={N}")
    m_gpu = _map_from_cells(cells, ranks_depth, ranks_feat)
    dense = np.repeat(np.arange(occ.size), lengths)               # occupied cells renumbered
    m_ref = _map_from_cells(dense, ranks_depth, ranks_feat)

    out = torch.full((n_cells, C), float("nan"), dtype=torch.float32, device=dev())
    dws.bevpool_forward(to_gpu(depth), to_gpu(feat), _gpu_map(m_gpu), n_cells, out=out)
    torch.cuda.synchronize()
    occ_t = torch.from_numpy(occ).to(dev())
    got = out.index_select(0, occ_t).cpu().numpy()
    out.index_fill_(0, occ_t, 0.0)
    assert not bool((out != 0).any()), "an empty cell is not 0 (or an element was not written)"
    del out
    torch.cuda.empty_cache()
    ref, ref_abs = oracle.forward(depth, feat, "f16", 1.0, C, m_ref, occ.size, with_abs=True)
    check_forward(got, ref, ref_abs, "f16", np.arange(occ.size), "largest output")


# More than 2^24 intervals: the short-role blocks (one interval per wave)
# exceed one launch's cap of 2^22 blocks and continue in a second launch.
# A small table keeps the plain block order; one over 8 MB takes the
# XCD-contiguous order, whose logical blocks then span both launches.
MANY = 17_000_000


@pytest.mark.parametrize("table_rows", [1000, 600_000], ids=["plain-order", "xcd-order"])
def test_forward_more_intervals_than_one_launch(table_rows):
    C = 8
    rng = np.random.default_rng(47)
    n_cells = MANY + 3_000_000
    occ = np.sort(rng.permutation(n_cells)[:MANY])
    lengths = rng.integers(1, 3, MANY)
    lengths[rng.integers(0, MANY, 20)] = 500                      # a few long intervals
    cells = np.repeat(occ, lengths)
    N = cells.size
    n_depth = 4096
    feat = rng.standard_normal((table_rows, C)).astype(np.float16)
    depth = rng.random(n_depth).astype(np.float16)
    say(f"[many intervals] intervals={MANY} points={N} table rows={table_rows}")
    m = _map_from_cells(cells, rng.integers(0, n_depth, N), rng.integers(0, table_rows, N))
    out = torch.full((n_cells, C), float("nan"), dtype=torch.float32, device=dev())
    dws.bevpool_forward(to_gpu(depth), to_gpu(feat), _gpu_map(m), n_cells, out=out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    del out
    torch.cuda.empty_cache()
    ref, ref_abs = oracle.forward(depth, feat, "f16", 1.0, C, m, n_cells, with_abs=True)
    check_forward(got, ref, ref_abs, "f16", m["ranks_bev"], f"many intervals rows={table_rows}")


def test_segment_reduce_more_segments_than_one_launch():
    # fp32 rows of 64 channels are 16 chunks, so segments over 384 points are
    # split four ways by channels (the part groups sit in the first launch)
    C = 64
    rng = np.random.default_rng(53)
    n_seg = MANY
    lens = (rng.random(n_seg) < 0.1).astype(np.int64)
    lens[rng.integers(0, n_seg, 10)] = 2000
    lens[-1] = 3                                                  # in the second launch
    offsets = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    N = int(offsets[-1])
    table = rng.standard_normal((5000, C)).astype(np.float32)
    idx = rng.integers(0, 5000, N).astype(np.int32)
    weights = rng.random(N).astype(np.float32)
    say(f"[many segments] segments={n_seg} points={N} C={C}")
    out = torch.full((n_seg, C), float("nan"), dtype=torch.float32, device=dev())
    dws.bevpool_segment_reduce(to_gpu(weights), to_gpu(table), to_gpu(idx), to_gpu(offsets),
                               out=out)
    torch.cuda.synchronize()
    # the oracle sees only the non-empty segments, renumbered densely (the
    # sums do not depend on the numbering); empty ones must be exactly zero
    full = np.flatnonzero(lens > 0)
    full_t = torch.from_numpy(full).to(dev())
    got = out.index_select(0, full_t).cpu().numpy().astype(np.float64)
    out.index_fill_(0, full_t, 0.0)
    assert not bool((out != 0).any()), "an empty segment is not 0 (or an element was not written)"
    del out
    torch.cuda.empty_cache()
    dense = np.concatenate([[0], np.cumsum(lens[full])]).astype(np.int32)
    ref, ref_abs = oracle.segment_reduce(weights, table, "f32", 1.0, idx, dense, with_abs=True)
    assert np.isfinite(got).all(), "an element was not written"
    assert (np.abs(got - ref) <= 1e-3 * ref_abs).all()


SEG_TABLES = [("f32", 64), ("f16", 64), ("f16", 80), ("e4m3", 128)]


@pytest.mark.parametrize("table_dtype,C", SEG_TABLES, ids=[f"{a}-C{b}" for a, b in SEG_TABLES])
def test_segment_reduce_largest_table(table_dtype, C):
    # a table at the byte limit, gathered at its top rows, through every row
    # geometry of the segment kernel: fp32 C=64 (split by channels), fp16
    # C=64 (staged rounds of 48 points), fp16 C=80 (staged rounds of 36
    # points, masked slots), e4m3 C=128 (16-byte chunks)
    eb = {"f32": 4, "f16": 2, "e4m3": 1}[table_dtype]
    n_rows = min(INT32_MAX // C, dws.MAX_TABLE_BYTES // (C * eb))
    say(f"[largest segment table {table_dtype} C={C}] rows={n_rows} bytes={n_rows * C * eb}")
    rng = np.random.default_rng(43 + C)
    used = np.unique(np.r_[np.arange(n_rows - 300, n_rows), rng.integers(0, n_rows, 100)])
    vals = rng.standard_normal((used.size, C))
    scale = 1.0
    if table_dtype == "f32":
        vals, tdt, wdt = vals.astype(np.float32), torch.float32, np.float32
    elif table_dtype == "f16":
        vals, tdt, wdt = vals.astype(np.float16), torch.float16, np.float16
    else:
        vals, scale = W.quantize_e4m3(vals.astype(np.float16))
        tdt, wdt = torch.uint8, np.float16
    lens = np.r_[rng.integers(0, 60, 40), [97, 400, 1500, 2000, 1, 0, 48, 49]]
    offsets = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    N = int(offsets[-1])
    pick = rng.integers(0, used.size, N).astype(np.int32)
    weights = rng.random(N).astype(wdt)
    table = torch.zeros((n_rows, C), dtype=tdt, device=dev())
    table[torch.from_numpy(used).to(dev())] = torch.from_numpy(vals).to(dev())
    out = torch.full((lens.size, C), float("nan"), dtype=torch.float32, device=dev())
    dws.bevpool_segment_reduce(to_gpu(weights), table, to_gpu(used[pick].astype(np.int32)),
                               to_gpu(offsets), table_scale=scale, out=out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    del table
    torch.cuda.empty_cache()
    ref, ref_abs = oracle.segment_reduce(weights, vals, table_dtype, scale, pick, offsets,
                                         with_abs=True)        # rows renumbered densely
    check_forward(got, ref, ref_abs, table_dtype, np.flatnonzero(lens > 0),
                  f"segment table {table_dtype} C={C}")


def test_build_map_largest_frustum():
    # n_img*D*H*W = 2^31 - 1, the largest frustum the map builder takes, with
    # kept points spread over it and packed into its last few thousand indices
    # (the last tile and the last emission block).
    P = INT32_MAX
    n_cells = 5000
    rng = np.random.default_rng(59)
    kept = np.unique(np.r_[rng.integers(0, P, 1_200_000), np.arange(P - 3000, P), [0, 1, 2]])
    cells = rng.integers(0, n_cells, kept.size).astype(np.int32)
    say(f"[largest frustum] P={P} kept={kept.size}")
    pc = torch.full((P,), -1, dtype=torch.int32, device=dev())
    pc[torch.from_numpy(kept).to(dev())] = torch.from_numpy(cells).to(dev())
    m = dws.bevpool_build_map(pc, 1, 1, 1, P, n_cells, capacity=kept.size)
    del pc
    torch.cuda.empty_cache()
    # The oracle sees only the kept points, renumbered 0..K-1 in order.  The
    # renumbering keeps their order, so the sorted order is the same; with one
    # image, one depth bin and one row the feature row of p is p itself.
    ref = oracle.build_map(cells, 1, 1, 1, kept.size, n_cells)
    got = map_to_numpy(m)
    assert got["n_points"] == ref["n_points"] == kept.size
    assert got["n_intervals"] == ref["n_intervals"]
    assert np.array_equal(got["ranks_depth"], kept[ref["ranks_depth"]])
    assert np.array_equal(got["ranks_feat"], kept[ref["ranks_feat"]])
    for k in ("ranks_bev", "interval_starts", "interval_lengths"):
        assert np.array_equal(got[k], ref[k]), k
