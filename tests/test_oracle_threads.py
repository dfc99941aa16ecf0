"""The all-core form of the oracle (used for the CPU baseline) must give the
single-thread oracle's result bit for bit: each thread takes whole intervals,
so every cell is summed by one thread in increasing t."""
import numpy as np
import pytest

import oracle
import workloads as W


@pytest.fixture(scope="module", autouse=True)
def _build():
    oracle.build(force=False)


def _same_bits(a, b):
    return np.array_equal(a.view(np.uint64), b.view(np.uint64))


@pytest.mark.parametrize("threads", [1, 2, 3, 7, 16, 64])
def test_threads_bitwise_on_headline_frame(threads):
    wl = W.make_workload(1)
    s = wl.spec
    m = oracle.build_map(wl.point_cell, s.n_img, s.D, s.H, s.W, s.n_cells)
    ref, ref_abs = oracle.forward(wl.depth, wl.feat, s.feat_dtype, wl.feat_scale, s.C, m,
                                  s.n_cells, with_abs=True)
    got, got_abs = oracle.forward_threads(wl.depth, wl.feat, s.feat_dtype, wl.feat_scale, s.C,
                                          m, s.n_cells, threads, with_abs=True)
    assert _same_bits(got, ref) and _same_bits(got_abs, ref_abs)


@pytest.mark.parametrize("seed", range(12))
def test_threads_bitwise_on_random_maps(seed):
    rng = np.random.default_rng(500 + seed)
    n_img, D, H, Wd = 1, int(rng.integers(1, 5)), int(rng.integers(1, 5)), int(rng.integers(1, 60))
    P = n_img * D * H * Wd
    n_cells = int(rng.choice([1, 3, 50, 4000]))
    pc = W.make_random_cells(rng, P, n_cells, p_drop=float(rng.choice([0.0, 0.5, 0.99])),
                             hot_cells=int(rng.choice([0, 2])))
    C = int(rng.choice([1, 8, 24]))
    dtype = str(rng.choice(["f32", "f16", "e4m3"]))
    depth = rng.random((n_img, D, H, Wd)).astype(np.float32 if dtype == "f32" else np.float16)
    feat = rng.standard_normal((n_img, H, Wd, C))
    scale = 1.0
    if dtype == "f32":
        feat = feat.astype(np.float32)
    elif dtype == "f16":
        feat = feat.astype(np.float16)
    else:
        feat, scale = W.quantize_e4m3(feat)
    m = oracle.build_map(pc, n_img, D, H, Wd, n_cells)
    ref = oracle.forward(depth, feat, dtype, float(scale), C, m, n_cells)
    for threads in (1, 2, 5, 1000):          # also more threads than intervals
        got = oracle.forward_threads(depth, feat, dtype, float(scale), C, m, n_cells, threads)
        assert _same_bits(got, ref), f"seed {seed}, {threads} threads"


def test_threads_reject_a_map_that_splits_a_cell():
    """Two intervals with the same cell would let two threads add into one
    cell: the threaded form refuses such a map (the plain oracle accepts any
    map, being the definition)."""
    m = {"ranks_depth": np.arange(4, dtype=np.int32), "ranks_feat": np.zeros(4, np.int32),
         "ranks_bev": np.array([0, 0, 1, 0], np.int32),
         "interval_starts": np.array([0, 2, 3], np.int32),
         "interval_lengths": np.array([2, 1, 1], np.int32)}
    depth, feat = np.ones(4, np.float32), np.ones((1, 2), np.float32)
    oracle.forward(depth, feat, "f32", 1.0, 2, m, 2)
    with pytest.raises(ValueError):
        oracle.forward_threads(depth, feat, "f32", 1.0, 2, m, 2, 2)
    gap = dict(m, ranks_bev=np.array([0, 0, 1, 2], np.int32),
               interval_starts=np.array([0, 3], np.int32), interval_lengths=np.array([2, 1], np.int32))
    with pytest.raises(ValueError):                          # intervals must tile the points
        oracle.forward_threads(depth, feat, "f32", 1.0, 2, gap, 3, 2)
