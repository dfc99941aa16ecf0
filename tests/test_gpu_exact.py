"""Exact-sum GPU parity: the HIP path must equal the oracle bit for bit.

Inputs are chosen so that every sum is exact in fp32 whatever the order of
summation, which removes rounding from the comparison:
  * features are nonzero integers in [-8, 8] (fp32, fp16, or e4m3 codes --
    e4m3 holds every integer up to 16 exactly -- with the power-of-two scale
    0.5);
  * depth values and segment weights are 0.5, 1 or 2 (or absent: 1).
Every term d * f (* 0.5) is then a nonzero multiple of 1/4 of magnitude at
most 16, so with at most 4,099 points per cell every partial sum is a
multiple of 1/4 below 2^17 in magnitude: 19 significant bits, exact in fp32's
24.  The oracle's fp64 sum is therefore the exact sum, and the kernel's fp32
sum must equal it exactly.  Because no term is zero, dropping or duplicating
any single point changes its cell's sum by at least 1/4 in every channel:
a lost or repeated point cannot pass (the scaled 1e-3 / 2e-2 bars of the
other parity tests can miss one point among hundreds).  Each test checks
these premises on its own inputs before comparing.

Coverage.  A feature row is split into G lane chunks (16 bytes; 8 bytes for
e4m3 rows under 256 bytes, 128 for segments).  The kernels have a compiled
wave geometry for G in {1, 2, 4, 5, 6, 8, 10, 12, 16, 20, 24, 32, 64}, and
every other G runs on a kernel with its points per wave (64 // G) fixed at
compile time: 21 (G=3), 9 (7), 7 (9), 5 (11), 4 (13-15), 3 (17-21), 2
(22-31), 1 (33-63).  The channel lists below take every compiled G and a
member of every points-per-wave class, for fp32, fp16 and both e4m3 chunk
sizes, in BEV pooling and in segment reductions (where rows of 16 or more
chunks, a multiple of 4, split long segments four ways by channels, and
long segments of other compiled rows stage extra loads in LDS).  Interval
lengths take every value from 1 to 99 -- every request round (at most 64
points), index batch (at most 64) and the one-wave limit (96) -- and then
values around 4x those (long intervals are split in quarters), around the
channel-split limit 384 and up to 1,440 points (BEV) or 4,099 (segments).
"""
import numpy as np
import pytest
import torch

import depth_weighted_scatter_amd as dws
import oracle
import workloads as W
from gpu_util import dev, feat_tensor, map_from_numpy, say, to_gpu

pytestmark = pytest.mark.gpu

SHORT = list(range(1, 100))
LONG_BEV = [101, 107, 108, 109, 127, 128, 129, 143, 144, 145, 191, 192, 193, 215, 216, 217,
            255, 256, 257, 383, 384, 385, 511, 512, 513, 1000, 1440]
LONG_SEG = [127, 128, 129, 191, 192, 193, 215, 216, 217, 255, 256, 257, 383, 384, 385, 386,
            600, 1001, 4099]

# (feature dtype, C).  G = chunks per row: fp32 C/4, fp16 C/8, e4m3 C/8 below
# 256 bytes or when not a multiple of 16 bytes, else C/16.
_G_LIST = [1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 16, 17, 20, 21, 22, 24, 31, 32, 33, 63, 64]
BEV_GEOMETRIES = ([("f32", 4 * g) for g in _G_LIST] + [("f16", 8 * g) for g in _G_LIST]
                  + [("e4m3", 8 * g) for g in _G_LIST if 8 * g < 256]          # 8-byte chunks
                  + [("e4m3", 264), ("e4m3", 504)]                              # 8-byte, G 33 / 63
                  + [("e4m3", 16 * g) for g in (16, 17, 20, 21, 22, 24, 32, 33, 63, 64)])
# Segments: 16-byte e4m3 chunks from 128-byte rows; long segments of 16-chunk
# (or wider, multiple-of-4) rows split four ways by channels.
SEG_GEOMETRIES = ([("f32", 4 * g) for g in (1, 2, 3, 4, 5, 7, 8, 10, 11, 12, 16, 17, 20, 24,
                                            32, 33, 64)]
                  + [("f16", 8 * g) for g in (1, 2, 3, 4, 5, 6, 7, 8, 10, 12, 16, 17, 20, 24,
                                              32, 33, 64)]
                  + [("e4m3", c) for c in (8, 40, 72, 80, 120, 136, 248)]       # 8-byte chunks
                  + [("e4m3", c) for c in (128, 144, 192, 256, 272, 320, 512, 528, 1024)])


@pytest.fixture(scope="module", autouse=True)
def _setup():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    oracle.build(force=False)
    dws._load()


def _ids(cases):
    return [f"{a}-C{b}" for a, b in cases]


def _premises(feat, feat_dtype, weights, ref):
    """The inputs hold no zero term, and the oracle's sums are exact fp32
    values: multiples of 1/4 below 2^22 in magnitude."""
    if feat_dtype == "e4m3":
        assert not np.isin(feat, [0x00, 0x80, 0x7F, 0xFF]).any(), "a zero or NaN e4m3 code"
    else:
        assert (feat != 0).all() and np.isfinite(feat).all()
    if weights is not None:
        assert (weights != 0).all() and np.isfinite(weights).all()
    q = ref * 4.0
    assert np.array_equal(q, np.round(q)), "oracle sums are not multiples of 1/4"
    assert float(np.abs(ref).max(initial=0.0)) < 2.0 ** 22
    assert np.array_equal(ref.astype(np.float32).astype(np.float64), ref)


def _bev_inputs(rng, feat_dtype, C, lengths, D=3):
    """A 1 x D x 1 x Wd frustum whose kept points form one interval per
    requested length (shuffled over the frustum, cells with gaps); D depth
    bins share each feature row, as in BEV pooling."""
    n_pts = int(sum(lengths))
    Wd = (n_pts + 16 + D - 1) // D
    P = D * Wd
    n_cells = 3 * len(lengths) + 7
    cells = rng.choice(n_cells, size=len(lengths), replace=False)
    pc = np.full(P, -1, np.int32)
    pc[rng.permutation(P)[:n_pts]] = np.repeat(cells, lengths).astype(np.int32)
    depth = W.power_of_two_weights(rng, P, "f32" if feat_dtype == "f32" else "f16")
    feat, scale = W.exact_values(rng, (Wd, C), feat_dtype)
    return pc, (1, D, 1, Wd), n_cells, depth, feat, scale


def _gpu_forward(depth, feat, scale, m, n_cells, C, out_dtype=torch.float32):
    out = torch.full((n_cells, C), float("nan"), dtype=out_dtype, device=dev())
    if out_dtype == torch.float32:
        dws.bevpool_forward(to_gpu(depth), feat_tensor(feat), m, n_cells, feat_scale=scale, out=out)
    else:
        dws.bevpool_forward_ex(to_gpu(depth), feat_tensor(feat), m, n_cells, out_dtype=out_dtype,
                               feat_scale=scale, out=out)
    torch.cuda.synchronize()
    return out.cpu()


def _assert_exact(got: torch.Tensor, ref: np.ndarray, label: str):
    g = got.to(torch.float64).numpy()
    if not np.array_equal(g, ref):
        bad = np.argwhere(g != ref)
        r, c = bad[0]
        raise AssertionError(f"{label}: {bad.shape[0]} elements differ, first at cell {r} "
                             f"channel {c}: got {g[r, c]!r}, exact {ref[r, c]!r}")


@pytest.mark.parametrize("feat_dtype,C", BEV_GEOMETRIES, ids=_ids(BEV_GEOMETRIES))
def test_forward_exact_every_geometry(feat_dtype, C):
    rng = np.random.default_rng(1000 + C * 3 + len(feat_dtype))
    lengths = SHORT + LONG_BEV
    pc, (n_img, D, H, Wd), n_cells, depth, feat, scale = _bev_inputs(rng, feat_dtype, C, lengths)
    say(f"[exact forward {feat_dtype} C={C}] points={sum(lengths)} intervals={len(lengths)}")
    ref_map = oracle.build_map(pc, n_img, D, H, Wd, n_cells)
    assert sorted(ref_map["interval_lengths"].tolist()) == sorted(lengths)
    ref = oracle.forward(depth, feat, feat_dtype, scale, C, ref_map, n_cells)
    _premises(feat, feat_dtype, depth, ref)
    got = _gpu_forward(depth, feat, scale, map_from_numpy(ref_map), n_cells, C)
    _assert_exact(got, ref, f"forward {feat_dtype} C={C}")


NARROW_CASES = [("f16", 80, torch.float16), ("f16", 80, torch.bfloat16),
                ("e4m3", 80, torch.float16), ("e4m3", 256, torch.bfloat16),
                ("f32", 32, torch.float16), ("f16", 56, torch.bfloat16),
                ("f16", 128, torch.float16), ("f16", 136, torch.float16)]


@pytest.mark.parametrize("feat_dtype,C,out_dtype", NARROW_CASES,
                         ids=[f"{a}-C{b}-{str(o).split('.')[-1]}" for a, b, o in NARROW_CASES])
def test_forward_ex_exact_rounding(feat_dtype, C, out_dtype):
    """fp16 / bf16 output: the exact fp32 sum rounded once, to nearest-even,
    must equal torch's rounding of the oracle's (exact) sum."""
    rng = np.random.default_rng(2000 + C + len(feat_dtype))
    lengths = SHORT + [101, 128, 193, 257, 385, 1000]
    pc, (n_img, D, H, Wd), n_cells, depth, feat, scale = _bev_inputs(rng, feat_dtype, C, lengths)
    say(f"[exact forward_ex {feat_dtype} C={C} -> {out_dtype}]")
    ref_map = oracle.build_map(pc, n_img, D, H, Wd, n_cells)
    ref = oracle.forward(depth, feat, feat_dtype, scale, C, ref_map, n_cells)
    _premises(feat, feat_dtype, depth, ref)
    assert float(np.abs(ref).max()) < 65504.0                # no fp16 overflow
    want = torch.from_numpy(ref.astype(np.float32)).to(out_dtype).to(torch.float64).numpy()
    got = _gpu_forward(depth, feat, scale, map_from_numpy(ref_map), n_cells, C, out_dtype)
    _assert_exact(got, want, f"forward_ex {feat_dtype} C={C} {out_dtype}")


@pytest.mark.parametrize("k,feat_dtype", [(1, "f16"), (1, "e4m3"), (3, "f16"), (4, "f16"),
                                          (10, "f16"), (6, "e4m3")])
def test_forward_exact_on_workload_maps(k, feat_dtype):
    """The workloads' own maps (their interval-length mix, the long-interval
    clusters near the cameras, the 4-frame batch whose table takes the
    per-XCD block order) with exact inputs of the workload's shape."""
    s = W.spec(k)
    wl = W.make_workload(k)
    rng = np.random.default_rng(3000 + k)
    depth = W.power_of_two_weights(rng, s.n_frustum, "f16")
    feat, scale = W.exact_values(rng, (s.n_feat_rows, s.C), feat_dtype)
    say(f"[exact workload {k} {s.name} {feat_dtype}] P={s.n_frustum}")
    ref_map = oracle.build_map(wl.point_cell, s.n_img, s.D, s.H, s.W, s.n_cells)
    ref = oracle.forward(depth, feat, feat_dtype, scale, s.C, ref_map, s.n_cells)
    _premises(feat, feat_dtype, depth, ref)
    got = _gpu_forward(depth, feat, scale, map_from_numpy(ref_map), s.n_cells, s.C)
    _assert_exact(got, ref, f"workload {k} {feat_dtype}")


def _seg_inputs(rng, table_dtype, C, lengths, weighted, rows=3000):
    off = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    idx = rng.integers(0, rows, size=max(int(off[-1]), 1)).astype(np.int32)
    table, scale = W.exact_values(rng, (rows, C), table_dtype)
    w = (W.power_of_two_weights(rng, idx.size, "f32" if table_dtype == "f32" else "f16")
         if weighted else None)
    return off, idx, table, scale, w


@pytest.mark.parametrize("table_dtype,C", SEG_GEOMETRIES, ids=_ids(SEG_GEOMETRIES))
def test_segment_reduce_exact_every_geometry(table_dtype, C):
    rng = np.random.default_rng(4000 + C * 3 + len(table_dtype))
    lengths = [0] + SHORT + LONG_SEG + [0, 1]
    weighted = C % 3 != 0                                     # some geometries unweighted
    off, idx, table, scale, w = _seg_inputs(rng, table_dtype, C, lengths, weighted)
    say(f"[exact segments {table_dtype} C={C}] segments={len(lengths)} N={int(off[-1])} "
        f"weighted={weighted}")
    ref = oracle.segment_reduce(w, table, table_dtype, scale, idx, off)
    _premises(table, table_dtype, w, ref)
    out = torch.full((len(lengths), C), float("nan"), dtype=torch.float32, device=dev())
    dws.bevpool_segment_reduce(to_gpu(w) if w is not None else None, to_gpu(table), to_gpu(idx),
                               to_gpu(off), table_scale=scale, out=out)
    torch.cuda.synchronize()
    _assert_exact(out.cpu(), ref, f"segments {table_dtype} C={C}")


# ---------------------------------------------------------------- random mixes
# Channel counts that reach every kind of kernel (compiled chunk counts and the
# points-per-wave classes, both e4m3 chunk sizes).
_RANDOM_C = {"f32": [4, 8, 12, 20, 28, 36, 44, 52, 64, 68, 84, 96, 128, 132, 188, 252, 256],
             "f16": [8, 16, 24, 40, 56, 72, 80, 88, 104, 120, 128, 136, 168, 192, 256, 264,
                     320, 400, 504, 512],
             "e4m3": [8, 16, 24, 40, 56, 72, 80, 96, 104, 128, 136, 176, 248, 256, 264, 272,
                      336, 384, 512, 528, 784, 1024]}


def _random_cells(rng, P, n_cells):
    """Point cells of several shapes: uniform, hot cells (long intervals),
    clusters with long gaps, one end of the grid, very sparse."""
    kind = int(rng.integers(0, 5))
    if kind == 0:
        pc = rng.integers(0, n_cells, P)
    elif kind == 1:
        pc = rng.choice(rng.integers(0, n_cells, 5), P)
    elif kind == 2:
        centres = rng.integers(0, n_cells, 4)
        pc = np.clip(centres[rng.integers(0, 4, P)] + rng.integers(-150, 150, P), 0, n_cells - 1)
    elif kind == 3:
        lo = int(rng.integers(0, max(1, n_cells - 400)))
        pc = rng.integers(lo, min(n_cells, lo + 400), P)
    else:
        pc = rng.choice(rng.integers(0, n_cells, max(1, P // 300)), P)
    pc = pc.astype(np.int32)
    pc[rng.random(P) < float(rng.choice([0.0, 0.2, 0.6]))] = -1
    return pc


def forward_exact_case(seed):
    """One random forward case on exact inputs: feature type, channel count,
    output type, frustum shape, cell pattern, and sometimes a feature table
    padded past 8 MB (the per-XCD block order); the map is built on the GPU
    and compared bit for bit, the output too (16-bit outputs against torch's
    rounding of the exact sum)."""
    from gpu_util import assert_maps_equal, gpu_map, map_to_numpy
    rng = np.random.default_rng(50_000 + seed)
    fdt = str(rng.choice(["f32", "f16", "e4m3"]))
    C = int(rng.choice(_RANDOM_C[fdt]))
    odt = [torch.float32, torch.float16, torch.bfloat16][int(rng.integers(0, 3))]
    n_img = int(rng.integers(1, 4))
    D, H, Wd = int(rng.integers(1, 20)), int(rng.integers(1, 9)), int(rng.integers(1, 60))
    P = n_img * D * H * Wd
    n_cells = int(rng.choice([1, 7, 300, 5000, 60000]))
    pc = _random_cells(rng, P, n_cells)
    rows = n_img * H * Wd
    eb = {"f32": 4, "f16": 2, "e4m3": 1}[fdt]
    pad = (9 << 20) // (C * eb) + 1 if rng.random() < 0.2 else 0
    depth = W.power_of_two_weights(rng, P, "f32" if fdt == "f32" else "f16")
    feat, scale = W.exact_values(rng, (rows + pad, C), fdt)
    say(f"[exact random forward {seed}] {fdt} C={C} out={str(odt).split('.')[-1]} "
        f"P={P} cells={n_cells} pad={pad}")
    ref_map = oracle.build_map(pc, n_img, D, H, Wd, n_cells)
    m = gpu_map(pc, n_img, D, H, Wd, n_cells)
    assert_maps_equal(map_to_numpy(m), ref_map, f"seed {seed}")
    ref = oracle.forward(depth, feat[:rows], fdt, scale, C, ref_map, n_cells)   # padding unread
    _premises(feat[:rows], fdt, depth, ref)
    want = torch.from_numpy(ref.astype(np.float32)).to(odt).to(torch.float64).numpy()
    got = _gpu_forward(depth, feat, scale, m, n_cells, C, odt)
    _assert_exact(got, want, f"random forward seed {seed}")


def segment_exact_case(seed):
    """One random segment-reduce case on exact inputs: table type and width,
    weighted or not, bag lengths from empty to past the channel-split limit."""
    rng = np.random.default_rng(60_000 + seed)
    tdt = str(rng.choice(["f32", "f16", "e4m3"]))
    C = int(rng.choice(_RANDOM_C[tdt]))
    n_seg = int(rng.integers(1, 400))
    kind = int(rng.integers(0, 3))
    if kind == 0:
        lens = rng.integers(0, 40, n_seg)
    elif kind == 1:
        lens = rng.geometric(1 / 20, n_seg)
        lens[rng.random(n_seg) < 0.05] = 0
    else:
        lens = rng.integers(0, 10, n_seg)
        lens[rng.integers(0, n_seg, 3)] = rng.integers(380, 1500, 3)
    lens = lens.astype(np.int64)
    off = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    rows = int(rng.integers(1, 5000))
    idx = rng.integers(0, rows, size=max(int(off[-1]), 1)).astype(np.int32)
    table, scale = W.exact_values(rng, (rows, C), tdt)
    w = (W.power_of_two_weights(rng, idx.size, "f32" if tdt == "f32" else "f16")
         if rng.random() < 0.7 else None)
    say(f"[exact random segments {seed}] {tdt} C={C} segments={n_seg} N={int(off[-1])} "
        f"weighted={w is not None}")
    ref = oracle.segment_reduce(w, table, tdt, scale, idx, off)
    _premises(table, tdt, w, ref)
    out = torch.full((n_seg, C), float("nan"), dtype=torch.float32, device=dev())
    dws.bevpool_segment_reduce(to_gpu(w) if w is not None else None, to_gpu(table), to_gpu(idx),
                               to_gpu(off), table_scale=scale, out=out)
    torch.cuda.synchronize()
    _assert_exact(out.cpu(), ref, f"random segments seed {seed}")


@pytest.mark.parametrize("seed", range(40))
def test_forward_exact_random_mix(seed):
    forward_exact_case(seed)


@pytest.mark.parametrize("seed", range(20))
def test_segment_reduce_exact_random_mix(seed):
    segment_exact_case(seed)


# Maps the builder would never emit: the forward assumes nothing of
# ranks_feat and ranks_depth beyond being indices into the tables, so a
# caller's own map -- rows and depth bins in any order, repeated inside one
# interval, shared between cells -- must pool exactly like the oracle.
HAND_MAP_CASES = [("f16", 80), ("e4m3", 80), ("f32", 8), ("f16", 256), ("e4m3", 256),
                  ("f16", 48), ("f32", 36)]


@pytest.mark.parametrize("feat_dtype,C", HAND_MAP_CASES, ids=_ids(HAND_MAP_CASES))
def test_forward_exact_on_hand_built_maps(feat_dtype, C):
    rng = np.random.default_rng(3000 + C + len(feat_dtype))
    lengths = np.array(SHORT + [101, 128, 200, 385, 700, 1440], dtype=np.int64)
    rng.shuffle(lengths)
    n_iv = lengths.size
    n_cells = 3 * n_iv + 11
    cells = np.sort(rng.choice(n_cells, size=n_iv, replace=False)).astype(np.int32)
    starts = np.concatenate([[0], np.cumsum(lengths)[:-1]]).astype(np.int32)
    N = int(lengths.sum())
    rows, n_depth = 37, 53                       # few rows and bins: heavy reuse
    ref_map = {"ranks_bev": np.repeat(cells, lengths).astype(np.int32),
               "ranks_feat": rng.integers(0, rows, size=N).astype(np.int32),
               "ranks_depth": rng.integers(0, n_depth, size=N).astype(np.int32),
               "interval_starts": starts, "interval_lengths": lengths.astype(np.int32),
               "n_points": N, "n_intervals": n_iv}
    depth = W.power_of_two_weights(rng, n_depth, "f32" if feat_dtype == "f32" else "f16")
    feat, scale = W.exact_values(rng, (rows, C), feat_dtype)
    say(f"[hand-built map {feat_dtype} C={C}] points={N} intervals={n_iv}")
    ref = oracle.forward(depth, feat, feat_dtype, scale, C, ref_map, n_cells)
    _premises(feat, feat_dtype, depth, ref)
    got = _gpu_forward(depth, feat, scale, map_from_numpy(ref_map), n_cells, C)
    _assert_exact(got, ref, f"hand-built map {feat_dtype} C={C}")
