"""Seeded random cases that mix the features the parametrized tests vary one
at a time: feature / depth / output types, channel counts, clustered and
sparse cells, intervals past the one-wave limit, long empty regions, and
(sometimes) a feature table padded past 8 MB so the XCD-contiguous block order
is taken.  Every case is checked against the oracle: the map bit-exact, the
pooled output within the scaled bound (widened by the output rounding for
16-bit outputs), every element written and empty cells exactly zero.
Segment reductions get the same treatment with random offsets."""
import numpy as np
import pytest
import torch

import depth_weighted_scatter_amd as dws
import oracle
import workloads as W
from gpu_util import TOL, dev, gpu_map, map_to_numpy, assert_maps_equal, say, to_gpu

pytestmark = pytest.mark.gpu

C_CHOICES = {"f32": [4, 8, 12, 24, 28, 32, 48, 60, 80, 96, 128, 256],
             "f16": [8, 16, 24, 48, 56, 72, 80, 88, 96, 128, 152, 192, 200, 256, 320, 512],
             "e4m3": [8, 16, 40, 72, 80, 96, 128, 192, 200, 256, 264, 384, 512, 528, 1024]}
OUT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
UNIT = {"f32": 0.0, "f16": 2.0 ** -11, "bf16": 2.0 ** -8}
TINY = {"f32": 0.0, "f16": 2.0 ** -25, "bf16": 2.0 ** -134}


@pytest.fixture(scope="module", autouse=True)
def _setup():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    oracle.build(force=False)
    dws._load()


def _cells(rng, P, n_cells):
    kind = int(rng.integers(0, 6))
    if kind == 0:                                        # uniform
        pc = rng.integers(0, n_cells, P)
    elif kind == 1:                                      # a few hot cells (long intervals)
        pc = rng.choice(rng.integers(0, n_cells, 5), P)
    elif kind == 2:                                      # clusters with long gaps between
        centres = rng.integers(0, n_cells, 4)
        pc = np.clip(centres[rng.integers(0, 4, P)] + rng.integers(-150, 150, P), 0, n_cells - 1)
    elif kind == 3:                                      # one end of the grid only
        lo = int(rng.integers(0, max(1, n_cells - 400)))
        pc = rng.integers(lo, min(n_cells, lo + 400), P)
    elif kind == 4:                                      # very sparse
        pc = rng.choice(rng.integers(0, n_cells, max(1, P // 300)), P)
    else:                                                # mixture
        pc = np.where(rng.random(P) < 0.5, rng.integers(0, n_cells, P),
                      rng.choice(rng.integers(0, n_cells, 3), P))
    pc = pc.astype(np.int32)
    pc[rng.random(P) < float(rng.choice([0.0, 0.2, 0.6]))] = -1
    return pc, kind


@pytest.mark.parametrize("seed", range(40))
def test_forward_random_mix(seed):
    rng = np.random.default_rng(9000 + seed)
    fdt = str(rng.choice(["f32", "f16", "e4m3"]))
    C = int(rng.choice(C_CHOICES[fdt]))
    odt = str(rng.choice(["f32", "f16", "bf16"]))
    n_img = int(rng.integers(1, 4))
    D, H, Wd = int(rng.integers(1, 20)), int(rng.integers(1, 9)), int(rng.integers(1, 60))
    P = n_img * D * H * Wd
    n_cells = int(rng.choice([1, 7, 300, 5000, 60000]))
    pc, kind = _cells(rng, P, n_cells)
    # feature rows: the image rows, sometimes with unused padding rows after
    # them so the table passes 8 MB (only the first n_img*H*Wd rows are read)
    rows = n_img * H * Wd
    eb = {"f32": 4, "f16": 2, "e4m3": 1}[fdt]
    pad_rows = 0
    if rng.random() < 0.25:
        pad_rows = (9 << 20) // (C * eb) + 1
    depth = rng.random(P)
    feat = rng.standard_normal((rows, C))
    scale = 1.0
    if fdt == "f32":
        depth, feat = depth.astype(np.float32), feat.astype(np.float32)
    elif fdt == "f16":
        depth, feat = depth.astype(np.float16), feat.astype(np.float16)
    else:
        depth = depth.astype(np.float16)
        feat, scale = W.quantize_e4m3(feat.astype(np.float16))
    say(f"[fuzz {seed}] {fdt} C={C} out={odt} P={P} cells={n_cells} kind={kind} pad={pad_rows}")
    ref = oracle.build_map(pc, n_img, D, H, Wd, n_cells)
    m = gpu_map(pc, n_img, D, H, Wd, n_cells)
    assert_maps_equal(map_to_numpy(m), ref, f"seed {seed}")
    out_ref, out_abs = oracle.forward(depth, feat, fdt, scale, C, ref, n_cells, with_abs=True)

    feat_t = torch.zeros((rows + pad_rows, C), dtype=torch.from_numpy(feat).dtype, device=dev())
    feat_t[:rows] = to_gpu(feat)
    out = torch.full((n_cells, C), float("nan"), dtype=OUT[odt], device=dev())
    dws.bevpool_forward_ex(to_gpu(depth), feat_t, m, n_cells, out_dtype=OUT[odt],
                           feat_scale=scale, out=out)
    torch.cuda.synchronize()
    got = out.to(torch.float64).cpu().numpy()
    assert np.isfinite(got).all(), "an element was not written"
    tol = TOL[fdt]
    bound = tol * out_abs + UNIT[odt] * (np.abs(out_ref) + tol * out_abs) + TINY[odt]
    assert (np.abs(got - out_ref) <= bound).all(), "error beyond the bound"
    empty = np.ones(n_cells, bool)
    empty[ref["ranks_bev"]] = False
    assert (got[empty] == 0).all(), "an empty cell is not zero"


@pytest.mark.parametrize("seed", range(16))
def test_segment_reduce_random_mix(seed):
    rng = np.random.default_rng(9500 + seed)
    tdt = str(rng.choice(["f32", "f16", "e4m3"]))
    C = int(rng.choice(C_CHOICES[tdt]))
    n_seg = int(rng.choice([1, 3, 100, 4000]))
    lens = rng.geometric(1.0 / float(rng.choice([1.5, 8, 40])), n_seg) - 1
    if rng.random() < 0.5:
        lens[rng.integers(0, n_seg, 2)] = int(rng.choice([97, 500, 3000]))
    lens[0] = max(lens[0], 1)                    # at least one point overall
    offsets = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    N = int(offsets[-1])
    n_rows = int(rng.choice([1, 50, 20000]))
    idx = rng.integers(0, n_rows, max(N, 1)).astype(np.int32)[:N]
    table = rng.standard_normal((n_rows, C))
    scale = 1.0
    weighted = bool(rng.random() < 0.7)
    if tdt == "f32":
        table, wdt = table.astype(np.float32), np.float32
    elif tdt == "f16":
        table, wdt = table.astype(np.float16), np.float16
    else:
        table, scale = W.quantize_e4m3(table.astype(np.float16))
        wdt = np.float16
    weights = rng.random(N).astype(wdt) if weighted else None
    say(f"[segment fuzz {seed}] {tdt} C={C} segments={n_seg} points={N} weighted={weighted}")
    ref, ref_abs = oracle.segment_reduce(weights, table, tdt, scale, idx, offsets, with_abs=True)
    out = torch.full((n_seg, C), float("nan"), dtype=torch.float32, device=dev())
    dws.bevpool_segment_reduce(to_gpu(weights) if weighted else None, to_gpu(table),
                               to_gpu(idx), to_gpu(offsets), table_scale=scale, out=out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    assert np.isfinite(got).all()
    assert (np.abs(got - ref) <= TOL[tdt] * ref_abs).all()
    assert (got[lens == 0] == 0).all()
