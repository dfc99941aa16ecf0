"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

The map must match bit for bit; the pooled output must be within the scaled
error bound (1e-3 for fp32/fp16 features, 2e-2 for e4m3, see gpu_util.TOL),
with empty cells exactly zero.  Inputs are the seeded synthetic workloads
plus small geometries that span several tiles with ragged tails.
"""
import numpy as np
import pytest
import torch

import depth_weighted_scatter_amd as dws
import oracle
import workloads as W
from gpu_util import (MAP_KEYS, assert_maps_equal, check_forward, gpu_forward, gpu_map,
                      map_from_numpy, map_to_numpy, oracle_reference, say, to_gpu)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _setup():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    oracle.build(force=False)
    dws._load()          # raises if the HIP library is not built


def _workload_case(k):
    wl = W.make_workload(k)
    s = wl.spec
    say(f"[workload {k} {s.name}] P={s.n_frustum} n_cells={s.n_cells} C={s.C} {s.feat_dtype}")
    ref = oracle.build_map(wl.point_cell, s.n_img, s.D, s.H, s.W, s.n_cells)
    return wl, s, ref


# ------------------------------------------------------------------ maps
@pytest.mark.parametrize("k", [0, 1, 2, 3, 4, 9])
def test_map_bit_exact_on_workloads(k):
    wl, s, ref = _workload_case(k)
    m = gpu_map(wl.point_cell, s.n_img, s.D, s.H, s.W, s.n_cells)
    assert_maps_equal(map_to_numpy(m), ref, f"workload {k}")


def _random_geometry(rng, P_max):
    n_img = int(rng.integers(1, 4))
    D = int(rng.integers(1, 9))
    H = int(rng.integers(1, 9))
    Wd = int(rng.integers(1, max(2, P_max // (n_img * D * H))))
    return n_img, D, H, Wd


@pytest.mark.parametrize("seed", range(12))
def test_map_bit_exact_random(seed):
    rng = np.random.default_rng(100 + seed)
    n_img, D, H, Wd = _random_geometry(rng, 40000)
    P = n_img * D * H * Wd
    n_cells = int(rng.choice([1, 2, 7, 300, 5000, 70000, 1 << 20, (1 << 31) - 1]))
    pc = W.make_random_cells(rng, P, min(n_cells, 1 << 30), p_drop=float(rng.choice([0, .3, .95])),
                             hot_cells=int(rng.choice([0, 1, 3])))
    say(f"[random map seed={seed}] P={P} geometry={(n_img, D, H, Wd)} n_cells={n_cells}")
    ref = oracle.build_map(pc, n_img, D, H, Wd, n_cells)
    got = map_to_numpy(gpu_map(pc, n_img, D, H, Wd, n_cells))
    assert_maps_equal(got, ref, f"seed {seed}")


@pytest.mark.parametrize("case", ["all_dropped", "one_point", "one_cell", "single_cell_grid",
                                  "tile_minus_1", "tile_plus_1", "last_cell_only",
                                  "cells_near_int32_max"])
def test_map_edge_cases(case):
    rng = np.random.default_rng(7)
    n_img, D, H, Wd, n_cells = 1, 1, 1, 5000, 64
    if case == "tile_minus_1":
        Wd = 2 * 2048 - 1
    elif case == "tile_plus_1":
        Wd = 2 * 2048 + 1
    P = n_img * D * H * Wd
    pc = W.make_random_cells(rng, P, n_cells, p_drop=0.2)
    if case == "all_dropped":
        pc[:] = -1
    elif case == "one_point":
        pc[:] = -1
        pc[P // 2] = 17
    elif case == "one_cell":
        pc[pc >= 0] = 31
    elif case == "single_cell_grid":
        n_cells = 1
        pc[pc >= 0] = 0
    elif case == "last_cell_only":
        pc[::3] = n_cells - 1
    elif case == "cells_near_int32_max":
        # the largest grid the map allows: every radix digit, the top one included
        n_cells = (1 << 31) - 1
        pc = rng.integers(n_cells - 3000, n_cells, P).astype(np.int32)
        pc[::7] = rng.integers(0, 1 << 16, pc[::7].size)
        pc[::11] = -1
    say(f"[map edge {case}] P={P} n_cells={n_cells}")
    ref = oracle.build_map(pc, n_img, D, H, Wd, n_cells)
    got = map_to_numpy(gpu_map(pc, n_img, D, H, Wd, n_cells))
    assert_maps_equal(got, ref, case)


def test_map_rejects_bad_cell_and_small_capacity():
    pc = np.array([0, 3, -1, 2, 1, 4], np.int32)
    say("[map errors] bad cell")
    with pytest.raises(dws.BevPoolError) as ei:
        gpu_map(pc, 1, 1, 1, 6, 4)
    assert ei.value.status == -6
    pc = np.array([0, 3, -1, 2, 1, 2], np.int32)
    say("[map errors] capacity")
    with pytest.raises(dws.BevPoolError) as ei:
        gpu_map(pc, 1, 1, 1, 6, 4, capacity=3)
    assert ei.value.status == -5
    m = gpu_map(pc, 1, 1, 1, 6, 4, capacity=5)
    assert m.n_points == 5 and m.n_intervals == 4


# --------------------------------------------------------------- forward
@pytest.mark.parametrize("k", [0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10])
def test_forward_on_workloads(k):
    wl, s, ref = _workload_case(k)
    m = gpu_map(wl.point_cell, s.n_img, s.D, s.H, s.W, s.n_cells)
    assert_maps_equal(map_to_numpy(m), ref, f"workload {k}")
    out_ref, out_abs = oracle_reference(wl.depth, wl.feat, s.feat_dtype, wl.feat_scale, s.C, ref,
                                        s.n_cells)
    say(f"  forward workload {k}")
    got = gpu_forward(wl.depth, wl.feat, wl.feat_scale, m, s.n_cells, s.C)
    check_forward(got, out_ref, out_abs, s.feat_dtype, ref["ranks_bev"], f"workload {k}")
    again = gpu_forward(wl.depth, wl.feat, wl.feat_scale, m, s.n_cells, s.C)
    assert np.array_equal(got.view(np.uint32), again.view(np.uint32)), "not deterministic"


def _make_inputs(rng, n_img, D, H, Wd, C, feat_dtype):
    depth = rng.random((n_img, D, H, Wd))
    depth /= depth.sum(axis=1, keepdims=True)
    feat = rng.standard_normal((n_img, H, Wd, C))
    scale = 1.0
    if feat_dtype == "f32":
        return depth.astype(np.float32), feat.astype(np.float32), scale
    if feat_dtype == "f16":
        return depth.astype(np.float16), feat.astype(np.float16), scale
    q, scale = W.quantize_e4m3(feat.astype(np.float16))
    return depth.astype(np.float16), q, float(scale)


# Chunk counts with a kernel of their own and others (7, 9, 11, 15, 19, 25,
# 33, 40 chunks: kernels with the points per wave fixed instead).
CHANNEL_CASES = [("f32", 4), ("f32", 8), ("f32", 12), ("f32", 24), ("f32", 28), ("f32", 48),
                 ("f32", 60), ("f32", 80), ("f32", 96), ("f32", 128), ("f32", 256),
                 ("f16", 8), ("f16", 24), ("f16", 48), ("f16", 56), ("f16", 64), ("f16", 72),
                 ("f16", 80), ("f16", 88), ("f16", 96), ("f16", 120), ("f16", 128), ("f16", 152),
                 ("f16", 192), ("f16", 200), ("f16", 256), ("f16", 320), ("f16", 512),
                 ("e4m3", 8), ("e4m3", 16), ("e4m3", 40), ("e4m3", 48), ("e4m3", 72), ("e4m3", 80),
                 ("e4m3", 96), ("e4m3", 128), ("e4m3", 192), ("e4m3", 200), ("e4m3", 256),
                 ("e4m3", 264), ("e4m3", 384), ("e4m3", 512), ("e4m3", 528), ("e4m3", 1024)]


@pytest.mark.parametrize("feat_dtype,C", CHANNEL_CASES, ids=[f"{a}-C{b}" for a, b in CHANNEL_CASES])
def test_forward_channel_widths(feat_dtype, C):
    rng = np.random.default_rng(C * 7 + len(feat_dtype))
    n_img, D, H, Wd, n_cells = 2, 6, 5, 37, 97
    P = n_img * D * H * Wd
    pc = W.make_random_cells(rng, P, n_cells, p_drop=0.3, hot_cells=2)
    depth, feat, scale = _make_inputs(rng, n_img, D, H, Wd, C, feat_dtype)
    say(f"[forward C={C} {feat_dtype}] P={P} n_cells={n_cells}")
    ref = oracle.build_map(pc, n_img, D, H, Wd, n_cells)
    m = gpu_map(pc, n_img, D, H, Wd, n_cells)
    assert_maps_equal(map_to_numpy(m), ref, "map")
    out_ref, out_abs = oracle_reference(depth, feat, feat_dtype, scale, C, ref, n_cells)
    got = gpu_forward(depth, feat, scale, m, n_cells, C)
    check_forward(got, out_ref, out_abs, feat_dtype, ref["ranks_bev"], f"C={C} {feat_dtype}")


@pytest.mark.parametrize("feat_dtype,C", [("f32", 8), ("f16", 80), ("e4m3", 80), ("f16", 128)])
def test_forward_length_one_intervals_bit_exact(feat_dtype, C):
    """One point per cell: out = d * f (* scale) with a single rounding, so
    the GPU must equal the oracle rounded to fp32 exactly."""
    rng = np.random.default_rng(11)
    n_img, D, H, Wd = 1, 4, 8, 16
    P = n_img * D * H * Wd
    n_cells = P + 13
    pc = rng.permutation(n_cells)[:P].astype(np.int32)
    pc[rng.random(P) < 0.25] = -1
    depth, feat, scale = _make_inputs(rng, n_img, D, H, Wd, C, feat_dtype)
    say(f"[length-1 {feat_dtype} C={C}]")
    ref = oracle.build_map(pc, n_img, D, H, Wd, n_cells)
    assert (ref["interval_lengths"] == 1).all()
    out_ref = oracle.forward(depth, feat, feat_dtype, scale, C, ref, n_cells)
    got = gpu_forward(depth, feat, scale, map_from_numpy(ref), n_cells, C)
    assert np.array_equal(got, out_ref.astype(np.float32))


@pytest.mark.parametrize("C", [80, 128])
def test_forward_length_two_intervals_bit_exact(C):
    """Two points per cell, fp16 inputs: each product d * f is exact in fp32
    and the two land in different slots of the owner, so the output is one
    fp32 addition of exact values, i.e. the exact sum rounded once to fp32 --
    what the oracle's fp64 sum (exact here) rounds to."""
    rng = np.random.default_rng(13)
    n_img, D, H, Wd = 1, 4, 8, 16
    P = n_img * D * H * Wd
    n_cells = P // 2 + 5
    cells = np.repeat(rng.permutation(n_cells)[:P // 2], 2).astype(np.int32)
    pc = rng.permutation(cells).astype(np.int32)
    depth, feat, scale = _make_inputs(rng, n_img, D, H, Wd, C, "f16")
    say(f"[length-2 f16 C={C}]")
    ref = oracle.build_map(pc, n_img, D, H, Wd, n_cells)
    assert (ref["interval_lengths"] == 2).all()
    out_ref = oracle.forward(depth, feat, "f16", scale, C, ref, n_cells)
    got = gpu_forward(depth, feat, scale, map_from_numpy(ref), n_cells, C)
    assert np.array_equal(got, out_ref.astype(np.float32))


def test_forward_e4m3_every_code():
    """All 254 finite e4m3 codes through the kernel's native fp8 decode."""
    C = 16
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    feat = np.zeros((16, 16, C), np.uint8)
    feat.reshape(-1)[:codes.size] = codes
    n_img, D, H, Wd = 1, 1, 16, 16                # 256 points; row(p) = p
    P = 256
    pc = np.arange(P, dtype=np.int32)              # one point per cell
    depth = np.ones((n_img, D, H, Wd), np.float16)
    scale = 0.5
    say("[e4m3 every code]")
    ref = oracle.build_map(pc, n_img, D, H, Wd, P)
    out_ref = oracle.forward(depth, feat, "e4m3", scale, C, ref, P)
    got = gpu_forward(depth, feat, scale, map_from_numpy(ref), P, C)
    assert np.array_equal(got, out_ref.astype(np.float32))
    dec = oracle.decode_e4m3(codes) * scale
    assert np.array_equal(got.reshape(-1)[:codes.size], dec.astype(np.float32))


@pytest.mark.parametrize("case", ["no_points", "one_long_interval", "long_and_short",
                                  "first_and_last_cell", "single_cell_grid"])
def test_forward_edge_cases(case):
    rng = np.random.default_rng(5)
    n_img, D, H, Wd, C, n_cells = 1, 8, 16, 40, 80, 300
    P = n_img * D * H * Wd
    pc = W.make_random_cells(rng, P, n_cells, p_drop=0.5)
    if case == "no_points":
        pc[:] = -1
    elif case == "one_long_interval":
        pc[pc >= 0] = 123                           # ~2500 points: many 64-point batches
    elif case == "long_and_short":
        pc[::2] = 7
    elif case == "first_and_last_cell":
        pc = np.where(pc >= 0, np.where(pc % 2 == 0, 0, n_cells - 1), -1).astype(np.int32)
    elif case == "single_cell_grid":
        n_cells = 1
        pc[pc >= 0] = 0
    depth, feat, scale = _make_inputs(rng, n_img, D, H, Wd, C, "f16")
    say(f"[forward edge {case}]")
    ref = oracle.build_map(pc, n_img, D, H, Wd, n_cells)
    m = gpu_map(pc, n_img, D, H, Wd, n_cells)
    assert_maps_equal(map_to_numpy(m), ref, case)
    out_ref, out_abs = oracle_reference(depth, feat, "f16", scale, C, ref, n_cells)
    got = gpu_forward(depth, feat, scale, m, n_cells, C)
    check_forward(got, out_ref, out_abs, "f16", ref["ranks_bev"], case)
    if case == "no_points":
        assert (got == 0).all()


GAP_CASES = ["head", "tail", "head_and_tail_one_cell", "interior_two_clusters",
             "many_interior_gaps", "gaps_around_chunk_sizes", "sparse_random", "half_rows_empty"]


@pytest.mark.parametrize("case", GAP_CASES)
def test_forward_large_empty_regions(case):
    """Maps with long runs of empty cells (grid wider than the occupied area,
    regions no point reaches, gaps of 255..513 cells around the 256-cell
    chunking): every empty cell must come out exactly 0 and every occupied
    cell must match the oracle."""
    rng = np.random.default_rng(100 + GAP_CASES.index(case))
    n_img, D, H, Wd, C = 1, 8, 16, 40, 16
    P = n_img * D * H * Wd
    n_cells = 60000
    if case == "head":
        pc = rng.integers(n_cells - 3000, n_cells, P)
    elif case == "tail":
        pc = rng.integers(0, 3000, P)
    elif case == "head_and_tail_one_cell":
        pc = np.full(P, 31337)
    elif case == "interior_two_clusters":
        pc = np.where(rng.random(P) < 0.5, rng.integers(0, 500, P), rng.integers(n_cells - 500, n_cells, P))
    elif case == "many_interior_gaps":
        base = rng.integers(0, 40, P) * 1500
        pc = base + rng.integers(0, 300, P)
    elif case == "gaps_around_chunk_sizes":
        # occupied cells separated by gaps of 255, 256, 257, 511, 512, 513, 1024 cells,
        # some starting on a chunk boundary
        edges, c = [], 100
        for g in [255, 256, 257, 511, 512, 513, 1024, 1, 300, 768]:
            edges.append(c)
            c += g + 1
        edges.append(1024 * 20)
        edges.append(1024 * 20 + 257)
        pc = rng.choice(np.array(edges), P)
    elif case == "sparse_random":
        pc = rng.choice(n_cells, 200, replace=False)[rng.integers(0, 200, P)]
    else:   # half_rows_empty: a 240 x 250 grid with rows 60..179 empty
        rows = rng.integers(0, 120, P)
        rows = np.where(rows >= 60, rows + 120, rows)
        pc = rows * 250 + rng.integers(0, 250, P)
    pc = pc.astype(np.int32)
    pc[rng.random(P) < 0.2] = -1
    depth, feat, scale = _make_inputs(rng, n_img, D, H, Wd, C, "f16")
    say(f"[forward large empty regions: {case}]")
    ref = oracle.build_map(pc, n_img, D, H, Wd, n_cells)
    m = gpu_map(pc, n_img, D, H, Wd, n_cells)
    assert_maps_equal(map_to_numpy(m), ref, case)
    out_ref, out_abs = oracle_reference(depth, feat, "f16", scale, C, ref, n_cells)
    got = gpu_forward(depth, feat, scale, m, n_cells, C)
    check_forward(got, out_ref, out_abs, "f16", ref["ranks_bev"], case)


def test_forward_graph_replay_matches_eager():
    """Captured forward calls replayed several times, with eager work and
    synchronisations in between; every replay must equal the eager result."""
    wl, s, ref = _workload_case(1)
    m = gpu_map(wl.point_cell, s.n_img, s.D, s.H, s.W, s.n_cells)
    depth, feat = to_gpu(wl.depth), to_gpu(wl.feat)
    eager = torch.empty((s.n_cells, s.C), dtype=torch.float32, device="cuda")
    dws.bevpool_forward(depth, feat, m, s.n_cells, out=eager)
    torch.cuda.synchronize()
    outs = [torch.full_like(eager, float("nan")) for _ in range(3)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):      # warm the binding on a side stream first
        dws.bevpool_forward(depth, feat, m, s.n_cells, out=outs[0])
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for o in outs:
            dws.bevpool_forward(depth, feat, m, s.n_cells, out=o)
    for rep in range(4):
        for o in outs:
            o.fill_(float("nan"))
        _ = (depth.float() * 2).sum()               # unrelated eager work
        torch.cuda.synchronize()
        say(f"  graph replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        for o in outs:
            assert torch.equal(o, eager), f"replay {rep} differs from eager"


def test_forward_ex_and_segment_reduce_graph_replay():
    """The narrow-output forward (on the batched frame, whose feature table
    takes the XCD-contiguous block order) and the segmented reduce, captured
    together and replayed with eager work between replays, match eager calls
    bit for bit."""
    wl, s, _ = _workload_case(4)
    m = gpu_map(wl.point_cell, s.n_img, s.D, s.H, s.W, s.n_cells)
    depth, feat = to_gpu(wl.depth), to_gpu(wl.feat)
    b = W.make_bags(1)
    w, t = to_gpu(b.weights), to_gpu(b.table)
    idx, off = to_gpu(b.indices), to_gpu(b.offsets)
    eager_f = dws.bevpool_forward_ex(depth, feat, m, s.n_cells, out_dtype=torch.float16)
    eager_b = dws.bevpool_segment_reduce(w, t, idx, off)
    torch.cuda.synchronize()
    out_f, out_b = torch.empty_like(eager_f), torch.empty_like(eager_b)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        dws.bevpool_forward_ex(depth, feat, m, s.n_cells, out_dtype=torch.float16, out=out_f)
        dws.bevpool_segment_reduce(w, t, idx, off, out=out_b)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        dws.bevpool_forward_ex(depth, feat, m, s.n_cells, out_dtype=torch.float16, out=out_f)
        dws.bevpool_segment_reduce(w, t, idx, off, out=out_b)
    for rep in range(3):
        out_f.fill_(float("nan"))
        out_b.fill_(float("nan"))
        _ = (t.float() * 2).sum()                   # unrelated eager work
        torch.cuda.synchronize()
        say(f"  graph replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_f.view(torch.int16), eager_f.view(torch.int16)), f"forward_ex replay {rep}"
        assert torch.equal(out_b.view(torch.int32), eager_b.view(torch.int32)), f"segments replay {rep}"


def test_forward_concurrent_streams_match_serial():
    """Calls on two streams at once (different maps and outputs) give the
    results of serial calls: the library keeps no state between calls."""
    wa, sa, _ = _workload_case(1)
    wb, sb, _ = _workload_case(3)
    ma = gpu_map(wa.point_cell, sa.n_img, sa.D, sa.H, sa.W, sa.n_cells)
    mb = gpu_map(wb.point_cell, sb.n_img, sb.D, sb.H, sb.W, sb.n_cells)
    da, fa, db, fb = to_gpu(wa.depth), to_gpu(wa.feat), to_gpu(wb.depth), to_gpu(wb.feat)
    ref_a = dws.bevpool_forward(da, fa, ma, sa.n_cells)
    ref_b = dws.bevpool_forward(db, fb, mb, sb.n_cells)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs_a = [torch.full_like(ref_a, float("nan")) for _ in range(4)]
    outs_b = [torch.full_like(ref_b, float("nan")) for _ in range(4)]
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    for oa, ob in zip(outs_a, outs_b):
        dws.bevpool_forward(da, fa, ma, sa.n_cells, out=oa, stream=s1)
        dws.bevpool_forward(db, fb, mb, sb.n_cells, out=ob, stream=s2)
    torch.cuda.synchronize()
    for oa, ob in zip(outs_a, outs_b):
        assert torch.equal(oa, ref_a) and torch.equal(ob, ref_b)


def _cells_with_lengths(rng, lengths, n_cells_extra=7, gaps=True):
    """point_cell for a 1 x 1 x 1 x P frustum whose kept points form one
    interval per requested length, in shuffled frustum order."""
    P = int(sum(lengths)) + 5
    n_cells = len(lengths) * (3 if gaps else 1) + n_cells_extra
    cells = rng.choice(n_cells, size=len(lengths), replace=False)
    pc = np.full(P, -1, np.int32)
    pos = rng.permutation(P)[:sum(lengths)]
    pc[pos] = np.repeat(cells, lengths).astype(np.int32)
    return pc, P, n_cells


LENGTH_CASES = [
    ("f16", 80, [1, 2, 63, 64, 65, 95, 96, 97, 127, 128, 129, 200, 411, 1000]),
    ("e4m3", 80, [1, 64, 65, 96, 97, 300, 1440]),
    ("f32", 8, [1, 30, 64, 65, 97, 500]),
    ("f16", 128, [64, 96, 97, 256, 700]),
    ("f16", 96, [5, 64, 97, 333]),            # runtime lane-count path (12 chunks)
    ("e4m3", 1024, [3, 97, 260]),             # 16-byte e4m3 chunks
]


@pytest.mark.parametrize("feat_dtype,C,lengths", LENGTH_CASES,
                         ids=[f"{a}-C{b}" for a, b, _ in LENGTH_CASES])
def test_forward_interval_length_boundaries(feat_dtype, C, lengths):
    """Intervals on both sides of the one-wave / long-interval split and of
    the 64-point index batches, in both block roles."""
    rng = np.random.default_rng(sum(lengths) + C)
    pc, P, n_cells = _cells_with_lengths(rng, lengths)
    n_img, D, H, Wd = 1, 1, 1, P
    depth, feat, scale = _make_inputs(rng, n_img, D, H, Wd, C, feat_dtype)
    say(f"[lengths {feat_dtype} C={C}] {lengths}")
    ref = oracle.build_map(pc, n_img, D, H, Wd, n_cells)
    assert sorted(ref["interval_lengths"].tolist()) == sorted(lengths)
    m = gpu_map(pc, n_img, D, H, Wd, n_cells)
    assert_maps_equal(map_to_numpy(m), ref, "map")
    out_ref, out_abs = oracle_reference(depth, feat, feat_dtype, scale, C, ref, n_cells)
    got = gpu_forward(depth, feat, scale, m, n_cells, C)
    check_forward(got, out_ref, out_abs, feat_dtype, ref["ranks_bev"], f"lengths {lengths}")


def test_forward_clustered_long_intervals():
    """Hundreds of long intervals next to each other (more than one per
    long-interval block), mixed with short ones, plus empty gaps."""
    rng = np.random.default_rng(21)
    lengths = list(rng.integers(97, 400, size=300)) + list(rng.integers(1, 60, size=3000))
    pc, P, n_cells = _cells_with_lengths(rng, [int(x) for x in lengths])
    n_img, D, H, Wd = 1, 1, 1, P
    depth, feat, scale = _make_inputs(rng, n_img, D, H, Wd, 80, "f16")
    say(f"[clustered long] P={P} intervals={len(lengths)}")
    ref = oracle.build_map(pc, n_img, D, H, Wd, n_cells)
    m = gpu_map(pc, n_img, D, H, Wd, n_cells)
    assert_maps_equal(map_to_numpy(m), ref, "map")
    out_ref, out_abs = oracle_reference(depth, feat, "f16", scale, 80, ref, n_cells)
    got = gpu_forward(depth, feat, scale, m, n_cells, 80)
    check_forward(got, out_ref, out_abs, "f16", ref["ranks_bev"], "clustered long")
    again = gpu_forward(depth, feat, scale, m, n_cells, 80)
    assert np.array_equal(got.view(np.uint32), again.view(np.uint32)), "not deterministic"


@pytest.mark.parametrize("k", [0, 1, 2, 3])
@pytest.mark.parametrize("order", [dws.ORDER_TILE_OUTER, dws.ORDER_DEPTH_OUTER],
                         ids=["tile_outer", "depth_outer"])
def test_baseline_orders_on_workloads(k, order):
    """The V2-style and V2+DO-style baselines compute the same pooled output."""
    wl, s, ref = _workload_case(k)
    out_ref, out_abs = oracle_reference(wl.depth, wl.feat, s.feat_dtype, wl.feat_scale, s.C, ref,
                                        s.n_cells)
    say(f"  baseline order {order} workload {k}")
    out = torch.full((s.n_cells, s.C), float("nan"), dtype=torch.float32, device="cuda")
    dws.bevpool_forward_baseline(order, to_gpu(wl.depth), to_gpu(wl.feat), map_from_numpy(ref),
                                 s.n_cells, feat_scale=wl.feat_scale, out=out)
    torch.cuda.synchronize()
    check_forward(out.cpu().numpy(), out_ref, out_abs, s.feat_dtype, ref["ranks_bev"],
                  f"baseline {order} workload {k}")



# ------------------------------------------------- segmented gather-reduce
def _gpu_segment_reduce(weights, table, scale, indices, offsets):
    n_seg, C = offsets.size - 1, table.shape[-1]
    out = torch.full((n_seg, C), float("nan"), dtype=torch.float32, device="cuda")
    dws.bevpool_segment_reduce(to_gpu(weights) if weights is not None else None, to_gpu(table),
                               to_gpu(indices), to_gpu(offsets), table_scale=scale, out=out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("k", [0, 1, 2, 3])
def test_segment_reduce_on_bag_workloads(k):
    b = W.make_bags(k)
    s = b.spec
    say(f"[bags {k} {s.name}] bags={s.n_bags} N={b.indices.size} C={s.C} {s.table_dtype}")
    ref, ref_abs = oracle.segment_reduce(b.weights, b.table, s.table_dtype, b.table_scale,
                                         b.indices, b.offsets, with_abs=True)
    got = _gpu_segment_reduce(b.weights, b.table, b.table_scale, b.indices, b.offsets)
    nonempty = np.nonzero(np.diff(b.offsets) > 0)[0]
    check_forward(got, ref, ref_abs, s.table_dtype, nonempty, f"bags {k}")
    again = _gpu_segment_reduce(b.weights, b.table, b.table_scale, b.indices, b.offsets)
    assert np.array_equal(got.view(np.uint32), again.view(np.uint32)), "not deterministic"


@pytest.mark.parametrize("case", ["all_empty", "one_long", "lengths_around_split",
                                  "unweighted_fp32", "leading_offset"])
def test_segment_reduce_edge_cases(case):
    rng = np.random.default_rng(33)
    rows, C = 50, 80
    table = rng.standard_normal((rows, C)).astype(np.float16)
    if case == "all_empty":
        lens = np.zeros(10, np.int64)
    elif case == "one_long":
        lens = np.array([3000])
    elif case == "lengths_around_split":
        lens = np.array([0, 1, 63, 64, 65, 95, 96, 97, 200, 0, 5])
    else:
        lens = rng.integers(0, 30, size=40)
    off = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    idx = rng.integers(0, rows, size=max(int(off[-1]), 1)).astype(np.int32)
    w = rng.random(idx.size).astype(np.float16)
    dtype = "f16"
    if case == "unweighted_fp32":
        table, w, dtype = table.astype(np.float32), None, "f32"
    if case == "leading_offset":                 # offsets need not start at 0
        off = off + 7
        idx = np.concatenate([rng.integers(0, rows, size=7).astype(np.int32), idx])
        w = np.concatenate([rng.random(7).astype(np.float16), w])
    say(f"[segment edge {case}] segments={off.size - 1} N={int(off[-1])}")
    ref, ref_abs = oracle.segment_reduce(w, table, dtype, 1.0, idx, off, with_abs=True)
    got = _gpu_segment_reduce(w, table, 1.0, idx, off)
    nonempty = np.nonzero(np.diff(off) > 0)[0]
    check_forward(got, ref, ref_abs, dtype, nonempty, case)


# Long segments of unsplit rows (2 to 12 chunks) take the long role with
# staged row loads; rows of 16 or more chunks (a multiple of 4) are split by
# channels.
# Lengths sit around the long-role threshold (96), the 64-point index batches
# a wave's quarter falls into, and the channel-split threshold (384).
LONG_SEGMENT_ROWS = [("f32", 8), ("f32", 16), ("f32", 20), ("f32", 32), ("f32", 40),
                     ("f16", 16), ("f16", 32), ("f16", 40), ("f16", 64), ("f16", 80),
                     ("f16", 128), ("f16", 256), ("e4m3", 80), ("e4m3", 128), ("f32", 24),
                     ("f16", 48), ("f16", 96), ("f16", 192), ("e4m3", 96), ("e4m3", 192),
                     ("f16", 56), ("f16", 88), ("f16", 200), ("e4m3", 72)]


@pytest.mark.parametrize("table_dtype,C", LONG_SEGMENT_ROWS,
                         ids=[f"{a}-C{b}" for a, b in LONG_SEGMENT_ROWS])
def test_segment_reduce_long_segment_lengths(table_dtype, C):
    rng = np.random.default_rng(61 + C)
    lens = np.array([97, 100, 127, 128, 129, 255, 256, 257, 259, 383, 384, 385, 386, 600,
                     1001, 4099, 3, 0, 96, 1])
    off = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    rows = 3000
    idx = rng.integers(0, rows, size=int(off[-1])).astype(np.int32)
    table = rng.standard_normal((rows, C))
    scale = 1.0
    if table_dtype == "f32":
        table, w = table.astype(np.float32), rng.random(idx.size).astype(np.float32)
    elif table_dtype == "f16":
        table, w = table.astype(np.float16), rng.random(idx.size).astype(np.float16)
    else:
        table, scale = W.quantize_e4m3(table.astype(np.float16))
        w = rng.random(idx.size).astype(np.float16)
    say(f"[long segments {table_dtype} C={C}] N={int(off[-1])}")
    ref, ref_abs = oracle.segment_reduce(w, table, table_dtype, scale, idx, off, with_abs=True)
    got = _gpu_segment_reduce(w, table, scale, idx, off)
    check_forward(got, ref, ref_abs, table_dtype, np.nonzero(lens > 0)[0],
                  f"long segments {table_dtype} C={C}")


# Row reads of the segmented reduce are bounded by the table's byte size (the
# raw buffer's range), so an index outside [0, n_rows) never reads memory
# outside the table: from n_rows up to 2^32 / row_bytes, and for small
# negatives, the row reads as zeros.  The expected values come from the
# oracle on the table with one zero row appended and those indices sent to it.
PAST_TABLE_ROWS = [("f16", 80), ("f16", 128), ("f16", 48), ("e4m3", 80), ("e4m3", 256),
                   ("f32", 8)]


@pytest.mark.parametrize("table_dtype,C", PAST_TABLE_ROWS,
                         ids=[f"{a}-C{b}" for a, b in PAST_TABLE_ROWS])
def test_segment_reduce_index_past_table_reads_zero(table_dtype, C):
    rng = np.random.default_rng(71 + C)
    rows = 500
    lens = np.array([1, 5, 18, 19, 54, 64, 97, 300, 500, 1000, 0, 2])
    off = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    n = int(off[-1])
    table = rng.standard_normal((rows, C))
    scale = 1.0
    if table_dtype == "f32":
        table, w = table.astype(np.float32), rng.random(n).astype(np.float32)
    elif table_dtype == "f16":
        table, w = table.astype(np.float16), rng.random(n).astype(np.float16)
    else:
        table, scale = W.quantize_e4m3(table.astype(np.float16))
        w = rng.random(n).astype(np.float16)
    row_bytes = table.dtype.itemsize * C
    idx = rng.integers(0, rows, size=n).astype(np.int64)
    past = np.array([rows, rows + 1, rows + 123, 1 << 20, (1 << 32) // row_bytes - 1, -1, -3])
    pick = rng.random(n) < 0.2
    idx[pick] = rng.choice(past, size=int(pick.sum()))
    assert idx.max() * row_bytes + row_bytes <= 1 << 32 and idx.min() * row_bytes >= -4096
    idx = idx.astype(np.int32)
    zero_row = np.zeros((1, C), dtype=table.dtype)
    table_ext = np.concatenate([table, zero_row])
    idx_ref = np.where((idx >= 0) & (idx < rows), idx, rows).astype(np.int32)
    say(f"[past-table indices {table_dtype} C={C}] N={n} out-of-range={int(pick.sum())}")
    ref, ref_abs = oracle.segment_reduce(w, table_ext, table_dtype, scale, idx_ref, off,
                                         with_abs=True)
    got = _gpu_segment_reduce(w, table, scale, idx, off)
    check_forward(got, ref, ref_abs, table_dtype, np.nonzero(lens > 0)[0],
                  f"past-table indices {table_dtype} C={C}")
