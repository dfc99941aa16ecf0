"""Checks that pin the CPU oracle to facts outside itself.

Each check raises AssertionError on failure.  They are shared by
test_oracle_pins.py (run against the real oracle) and test_oracle_mutants.py
(run against deliberately broken copies of the oracle, each of which must be
caught by at least one check).

What pins what:
  * fp16 decode   -- all 65536 codes vs numpy's float16 -> float64 cast.
  * e4m3 decode   -- all 256 codes vs torch.float8_e4m3fn, plus values the
                     OCP 8-bit float spec fixes (max 448, min normal 2^-6,
                     min subnormal 2^-9, NaN at S.1111.111).
  * map           -- a hand-worked example (tests/golden/hand_example.json);
                     numpy.lexsort on random micro-geometries with rows from
                     numpy.unravel_index / ravel_multi_index; structural
                     invariants on the synthetic workloads.
  * forward       -- the hand-worked example; a dense one-hot matrix product
                     built straight from point_cell (no map); closed forms
                     (all-ones inputs give point counts; integer features
                     give exact integer sums); invariants (total sum,
                     empty cells, linearity, permutation within a cell).
"""
from __future__ import annotations

import json
import os

import numpy as np
import torch

import oracle
import workloads as W

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ---------------------------------------------------------------- decoders
def check_f16_decode_all_codes():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.decode_f16(codes)
    ref = codes.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan), "fp16 NaN pattern differs"
    assert np.array_equal(got[~nan], ref[~nan]), "fp16 decode differs from numpy"
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan])), "fp16 sign of zero"


def check_e4m3_decode_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    got = oracle.decode_e4m3(codes)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan), "e4m3 NaN pattern differs from torch"
    assert np.array_equal(got[~nan], ref[~nan]), "e4m3 decode differs from torch"
    # values fixed by the OCP 8-bit floating point specification (E4M3)
    assert got[0x7E] == 448.0 and got[0xFE] == -448.0
    assert got[0x08] == 2.0 ** -6 and got[0x01] == 2.0 ** -9 and got[0x07] == 7 * 2.0 ** -9
    assert got[0x38] == 1.0 and got[0xB8] == -1.0 and got[0x39] == 1.125
    assert np.isnan(got[0x7F]) and np.isnan(got[0xFF]) and got[0x78] == 256.0
    assert nan.sum() == 2


# --------------------------------------------------------------- map pins
def _golden():
    with open(os.path.join(GOLDEN, "hand_example.json")) as f:
        return json.load(f)


def check_map_hand_example():
    g = _golden()
    geo = g["geometry"]
    m = oracle.build_map(np.array(g["point_cell"], np.int32), geo["n_img"], geo["D"], geo["H"],
                         geo["W"], geo["n_cells"])
    for k, v in g["expect_map"].items():
        assert m[k].tolist() == v, f"{k}: {m[k].tolist()} != {v}"
    assert m["n_points"] == 6 and m["n_intervals"] == 3


def lexsort_map(point_cell, n_img, D, H, W):
    """Independent map: numpy.lexsort by (cell, p); rows via unravel/ravel."""
    p = np.nonzero(point_cell >= 0)[0]
    cell = point_cell[p].astype(np.int64)
    order = np.lexsort((p, cell))          # primary key cell, ties by p
    p, cell = p[order], cell[order]
    img, d, h, w = np.unravel_index(p, (n_img, D, H, W))
    row = np.ravel_multi_index((img, h, w), (n_img, H, W))
    change = np.ones(cell.size, bool)
    change[1:] = cell[1:] != cell[:-1]
    starts = np.nonzero(change)[0]
    lengths = np.diff(np.append(starts, cell.size))
    return {"ranks_depth": p, "ranks_feat": row, "ranks_bev": cell,
            "interval_starts": starts, "interval_lengths": lengths}


def check_map_vs_lexsort(n_cases=40, seed=1):
    rng = np.random.default_rng(seed)
    for case in range(n_cases):
        n_img, D, H, W_ = (int(x) for x in rng.integers(1, 5, size=4))
        n_cells = int(rng.integers(1, 12))
        P = n_img * D * H * W_
        pc = W.make_random_cells(rng, P, n_cells, p_drop=float(rng.choice([0.0, 0.3, 0.9])),
                                 hot_cells=int(rng.integers(0, 3)))
        m = oracle.build_map(pc, n_img, D, H, W_, n_cells)
        ref = lexsort_map(pc, n_img, D, H, W_)
        for k in ref:
            assert np.array_equal(m[k], ref[k]), f"case {case}: {k} differs from lexsort"


def check_map_invariants(m, point_cell, n_img, D, H, W_, n_cells):
    rb, rd, rf = m["ranks_bev"], m["ranks_depth"], m["ranks_feat"]
    st, ln = m["interval_starts"], m["interval_lengths"]
    N, I = m["n_points"], m["n_intervals"]
    kept = np.nonzero(point_cell >= 0)[0]
    assert N == kept.size and rb.size == N and st.size == I
    assert int(ln.sum()) == N, "lengths do not sum to the kept count"
    if N:
        assert st[0] == 0 and (ln >= 1).all()
        assert np.array_equal(st[1:], st[:-1] + ln[:-1]), "intervals not contiguous"
        owner = np.repeat(np.arange(I), ln)
        assert np.array_equal(rb, rb[st][owner]), "ranks_bev not constant in an interval"
        assert (np.diff(rb[st]) > 0).all(), "interval cells not strictly increasing"
        assert ((rb >= 0) & (rb < n_cells)).all()
    # multiset of (cell, p) equals the kept frustum points; p unique
    assert np.array_equal(np.sort(rd), kept), "ranks_depth is not the kept point set"
    assert np.array_equal(rb, point_cell[rd]), "ranks_bev is not the cell of ranks_depth"
    img, d, h, w = np.unravel_index(rd, (n_img, D, H, W_))
    assert np.array_equal(rf, np.ravel_multi_index((img, h, w), (n_img, H, W_))), "ranks_feat row"


def check_map_invariants_on_workloads(keys=(0, 1)):
    for k in keys:
        wl = W.make_workload(k)
        s = wl.spec
        m = oracle.build_map(wl.point_cell, s.n_img, s.D, s.H, s.W, s.n_cells)
        check_map_invariants(m, wl.point_cell, s.n_img, s.D, s.H, s.W, s.n_cells)


# ----------------------------------------------------------- forward pins
def _values(arr, dtype, scale=1.0):
    """Decode stored values with numpy / torch (never the oracle)."""
    if dtype == "e4m3":
        t = torch.from_numpy(np.ascontiguousarray(arr)).view(torch.float8_e4m3fn)
        return t.to(torch.float64).numpy() * float(scale)
    return np.asarray(arr).astype(np.float64)


def dense_reference(point_cell, depth, feat, feat_dtype, scale, n_img, D, H, W_, C, n_cells):
    """out = M @ V with M the one-hot [cell, p] matrix, V[p] = depth[p] * feat[row(p)]."""
    P = point_cell.size
    dflat = _values(depth, "f", 1.0).reshape(-1)
    fmat = _values(feat, feat_dtype, scale).reshape(-1, C)
    img, d, h, w = np.unravel_index(np.arange(P), (n_img, D, H, W_))
    rows = np.ravel_multi_index((img, h, w), (n_img, H, W_))
    V = dflat[:, None] * fmat[rows]
    M = np.zeros((n_cells, P))
    keep = point_cell >= 0
    M[point_cell[keep], np.nonzero(keep)[0]] = 1.0
    return M @ V


def check_forward_hand_example():
    g = _golden()
    geo = g["geometry"]
    m = oracle.build_map(np.array(g["point_cell"], np.int32), geo["n_img"], geo["D"], geo["H"],
                         geo["W"], geo["n_cells"])
    out = oracle.forward(np.array(g["depth"], np.float32), np.array(g["feat"], np.float32), "f32",
                         1.0, geo["C"], m, geo["n_cells"])
    assert np.array_equal(out, np.array(g["expect_out"])), out


def _random_case(rng, feat_dtype):
    n_img, D, H, W_ = (int(x) for x in rng.integers(1, 5, size=4))
    C = int(rng.choice([1, 3, 8]))
    n_cells = int(rng.integers(1, 10))
    P = n_img * D * H * W_
    pc = W.make_random_cells(rng, P, n_cells, p_drop=0.25, hot_cells=int(rng.integers(0, 2)))
    depth = rng.random((n_img, D, H, W_))
    feat = rng.standard_normal((n_img, H, W_, C))
    scale = 1.0
    if feat_dtype == "f32":
        depth, feat = depth.astype(np.float32), feat.astype(np.float32)
    elif feat_dtype == "f16":
        depth, feat = depth.astype(np.float16), feat.astype(np.float16)
    else:
        depth = depth.astype(np.float16)
        feat, scale = W.quantize_e4m3(feat)
    return pc, depth, feat, float(scale), (n_img, D, H, W_, C, n_cells)


def check_forward_vs_dense(n_cases=30, seed=2):
    rng = np.random.default_rng(seed)
    for case in range(n_cases):
        fdt = ("f32", "f16", "e4m3")[case % 3]
        pc, depth, feat, scale, (n_img, D, H, W_, C, n_cells) = _random_case(rng, fdt)
        m = oracle.build_map(pc, n_img, D, H, W_, n_cells)
        out = oracle.forward(depth, feat, fdt, scale, C, m, n_cells)
        ref = dense_reference(pc, depth, feat, fdt, scale, n_img, D, H, W_, C, n_cells)
        assert np.allclose(out, ref, rtol=1e-12, atol=1e-12), f"case {case} ({fdt}) differs from dense"
    # the Tiny workload end to end
    wl = W.make_workload(0)
    s = wl.spec
    m = oracle.build_map(wl.point_cell, s.n_img, s.D, s.H, s.W, s.n_cells)
    out = oracle.forward(wl.depth, wl.feat, "f32", 1.0, s.C, m, s.n_cells)
    ref = dense_reference(wl.point_cell, wl.depth, wl.feat, "f32", 1.0, s.n_img, s.D, s.H, s.W,
                          s.C, s.n_cells)
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-12), "tiny workload differs from dense"


def check_forward_closed_forms(seed=3):
    rng = np.random.default_rng(seed)
    n_img, D, H, W_, C, n_cells = 2, 3, 4, 5, 6, 7
    P = n_img * D * H * W_
    pc = W.make_random_cells(rng, P, n_cells, p_drop=0.3, hot_cells=1)
    m = oracle.build_map(pc, n_img, D, H, W_, n_cells)
    counts = np.bincount(pc[pc >= 0], minlength=n_cells).astype(np.float64)
    # all-ones inputs: every channel of a cell is its point count
    ones_d = np.ones((n_img, D, H, W_), np.float16)
    out = oracle.forward(ones_d, np.ones((n_img, H, W_, C), np.float16), "f16", 1.0, C, m, n_cells)
    assert np.array_equal(out, np.repeat(counts[:, None], C, axis=1))
    # unit depth, integer features: exact integer sums of the features
    fi = rng.integers(-8, 9, size=(n_img, H, W_, C)).astype(np.float16)
    out = oracle.forward(ones_d, fi, "f16", 1.0, C, m, n_cells)
    img, d, h, w = np.unravel_index(np.arange(P), (n_img, D, H, W_))
    rows = np.ravel_multi_index((img, h, w), (n_img, H, W_))
    ref = np.zeros((n_cells, C))
    fflat = fi.reshape(-1, C).astype(np.float64)
    for p in range(P):                      # brute force over the tiny frustum
        if pc[p] >= 0:
            ref[pc[p]] += fflat[rows[p]]
    assert np.array_equal(out, ref)
    # e4m3 with a power-of-two scale: codes 0x38 (1.0) times scale 0.25
    q = np.full((n_img, H, W_, C), 0x38, np.uint8)
    out = oracle.forward(ones_d, q, "e4m3", 0.25, C, m, n_cells)
    assert np.array_equal(out, 0.25 * np.repeat(counts[:, None], C, axis=1))


def check_forward_invariants(seed=4):
    rng = np.random.default_rng(seed)
    for fdt in ("f32", "f16", "e4m3"):
        pc, depth, feat, scale, (n_img, D, H, W_, C, n_cells) = _random_case(rng, fdt)
        m = oracle.build_map(pc, n_img, D, H, W_, n_cells)
        out, out_abs = oracle.forward(depth, feat, fdt, scale, C, m, n_cells, with_abs=True)
        dv = _values(depth, "f").reshape(-1)
        fv = _values(feat, fdt, scale).reshape(-1, C)
        tot = sum(dv[p] * fv[r].sum() for p, r in zip(m["ranks_depth"], m["ranks_feat"]))
        assert abs(out.sum() - tot) <= 1e-9 * max(1.0, np.abs(out_abs).sum())
        empty = np.setdiff1d(np.arange(n_cells), m["ranks_bev"])
        assert (out[empty] == 0).all() and (out_abs[empty] == 0).all()
        assert (out_abs >= np.abs(out) - 1e-12).all()
        # linearity in depth (x2 is exact in every format)
        out2 = oracle.forward((depth * 2).astype(depth.dtype), feat, fdt, scale, C, m, n_cells)
        assert np.array_equal(out2, 2 * out)
        # permuting points inside each interval changes only rounding
        perm = np.arange(m["n_points"])
        for s0, ln in zip(m["interval_starts"], m["interval_lengths"]):
            perm[s0:s0 + ln] = s0 + rng.permutation(ln)
        mp = {k: (v[perm] if k.startswith("ranks") else v) for k, v in m.items()}
        outp = oracle.forward(depth, feat, fdt, scale, C, mp, n_cells)
        assert np.allclose(outp, out, rtol=0, atol=1e-12 * max(1.0, out_abs.max()))


def check_bad_cell_rejected():
    pc = np.array([0, 5, -1, 1], np.int32)
    try:
        oracle.build_map(pc, 1, 1, 1, 4, 5)
    except ValueError:
        pass
    else:
        raise AssertionError("cell == n_cells was accepted")
    try:
        oracle.build_map(np.array([0, -2, 1, 1], np.int32), 1, 1, 1, 4, 5)
    except ValueError:
        pass
    else:
        raise AssertionError("cell -2 was accepted")


# ------------------------------------------------- segmented gather-reduce
def check_segment_reduce_vs_embedding_bag(n_cases=12, seed=5):
    """Against torch.nn.functional.embedding_bag (mode sum, per-sample
    weights) in float64 -- a library routine with the same definition."""
    rng = np.random.default_rng(seed)
    for case in range(n_cases):
        rows, C, n_seg = int(rng.integers(1, 40)), int(rng.choice([1, 4, 16])), int(rng.integers(1, 30))
        lens = rng.integers(0, 12, size=n_seg)
        off = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        N = int(off[-1])
        idx = rng.integers(0, rows, size=N).astype(np.int32)
        fdt = ("f32", "f16", "e4m3")[case % 3]
        table = rng.standard_normal((rows, C))
        scale = 1.0
        if fdt == "f32":
            table = table.astype(np.float32)
        elif fdt == "f16":
            table = table.astype(np.float16)
        else:
            table, scale = W.quantize_e4m3(table)
        w = rng.random(N).astype(np.float16) if case % 2 else None
        got = oracle.segment_reduce(w, table, fdt, scale, idx, off)
        tv = torch.from_numpy(_values(table, fdt, scale).reshape(rows, C))
        psw = torch.from_numpy(w.astype(np.float64)) if w is not None else None
        ref = torch.nn.functional.embedding_bag(torch.from_numpy(idx.astype(np.int64)), tv,
                                                torch.from_numpy(off[:-1].astype(np.int64)),
                                                mode="sum", per_sample_weights=psw).numpy()
        assert np.allclose(got, ref, rtol=1e-12, atol=1e-12), f"case {case} differs from embedding_bag"


def check_segment_reduce_is_bev_forward():
    """The BEV forward is the segmented reduce with indices = ranks_feat,
    weights = depth[ranks_depth] and one segment per cell (empty cells are
    empty segments)."""
    rng = np.random.default_rng(9)
    pc, depth, feat, scale, (n_img, D, H, W_, C, n_cells) = _random_case(rng, "f16")
    m = oracle.build_map(pc, n_img, D, H, W_, n_cells)
    out = oracle.forward(depth, feat, "f16", scale, C, m, n_cells)
    counts = np.bincount(m["ranks_bev"], minlength=n_cells)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    w = depth.reshape(-1)[m["ranks_depth"]]
    seg = oracle.segment_reduce(w, feat.reshape(-1, C), "f16", scale, m["ranks_feat"], off)
    assert np.array_equal(seg, out)


ALL_CHECKS = [
    check_f16_decode_all_codes, check_e4m3_decode_all_codes,
    check_map_hand_example, check_map_vs_lexsort, check_map_invariants_on_workloads,
    check_forward_hand_example, check_forward_vs_dense, check_forward_closed_forms,
    check_forward_invariants, check_bad_cell_rejected,
    check_segment_reduce_vs_embedding_bag, check_segment_reduce_is_bev_forward,
]
