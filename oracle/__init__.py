"""CPU oracle for BEV pooling -- TEST INFRASTRUCTURE ONLY.

A thin ctypes wrapper over bevpool_oracle.c (plain C, double precision).
Only tests/, __graft_entry__.smoke() and the benchmark's cpu_baseline leg
use this package; the product library (depth_weighted_scatter_amd) never
imports it, and nothing here imports the product.

What it computes, and which passages of "Accelerating BEV Pooling on NVIDIA
GPUs for Physical AI Applications" each step follows, is documented in the
C source.  Every function here is pinned by tests/test_oracle_pins.py.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "bevpool_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libbevpool_oracle.so")

F32, F16, E4M3 = 0, 1, 2
_DTYPE_CODE = {"f32": F32, "f16": F16, "e4m3": E4M3}

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into oracle/libbevpool_oracle.so."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared",
                               "-Wall", "-Wextra", "-pthread", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _bind(path: str):
    lib = ctypes.CDLL(path)
    i64, vp, dp = ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p
    lib.oracle_decode_f16.restype = ctypes.c_double
    lib.oracle_decode_f16.argtypes = [ctypes.c_uint16]
    lib.oracle_decode_e4m3.restype = ctypes.c_double
    lib.oracle_decode_e4m3.argtypes = [ctypes.c_uint8]
    lib.oracle_build_map.restype = ctypes.c_int
    lib.oracle_build_map.argtypes = [vp, i64, i64, i64, i64, i64,
                                     vp, vp, vp, vp, vp,
                                     ctypes.POINTER(i64), ctypes.POINTER(i64)]
    lib.oracle_forward.restype = ctypes.c_int
    lib.oracle_forward.argtypes = [vp, ctypes.c_int, i64, vp, ctypes.c_int, i64, i64,
                                   ctypes.c_double, vp, vp, vp, i64, i64, dp, dp]
    lib.oracle_forward_threads.restype = ctypes.c_int
    lib.oracle_forward_threads.argtypes = [vp, ctypes.c_int, i64, vp, ctypes.c_int, i64, i64,
                                           ctypes.c_double, vp, vp, vp, i64, vp, vp, i64, i64,
                                           ctypes.c_int, dp, dp]
    lib.oracle_segment_reduce.restype = ctypes.c_int
    lib.oracle_segment_reduce.argtypes = [vp, ctypes.c_int, vp, ctypes.c_int, i64, i64,
                                          ctypes.c_double, vp, vp, i64, dp, dp]
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        _lib = _bind(_LIB_PATH)
    return _lib


def use_library(path):
    """Swap the loaded oracle build (the mutation tests load broken copies).

    Returns the previous handle; pass it back to restore.
    """
    global _lib
    prev = _load()
    _lib = _bind(path) if isinstance(path, str) else path
    return prev


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def decode_f16(codes) -> np.ndarray:
    lib = _load()
    c = np.asarray(codes, dtype=np.uint16).ravel()
    return np.array([lib.oracle_decode_f16(int(x)) for x in c], dtype=np.float64)


def decode_e4m3(codes) -> np.ndarray:
    lib = _load()
    c = np.asarray(codes, dtype=np.uint8).ravel()
    return np.array([lib.oracle_decode_e4m3(int(x)) for x in c], dtype=np.float64)


def build_map(point_cell: np.ndarray, n_img: int, D: int, H: int, W: int, n_cells: int) -> dict:
    """The five INT32 arrays for point_cell (int32 [n_img*D*H*W], -1 = dropped)."""
    lib = _load()
    pc = np.ascontiguousarray(point_cell, dtype=np.int32)
    P = n_img * D * H * W
    if pc.size != P:
        raise ValueError(f"point_cell has {pc.size} entries, expected {P}")
    cap = max(int((pc >= 0).sum()), 1)
    rd, rf, rb, st, ln = (np.empty(cap, np.int32) for _ in range(5))
    n_pts, n_iv = ctypes.c_int64(), ctypes.c_int64()
    rc = lib.oracle_build_map(_ptr(pc), n_img, D, H, W, n_cells,
                              _ptr(rd), _ptr(rf), _ptr(rb), _ptr(st), _ptr(ln),
                              ctypes.byref(n_pts), ctypes.byref(n_iv))
    if rc != 0:
        raise ValueError(f"oracle_build_map failed ({rc})")
    N, I = n_pts.value, n_iv.value
    return {"ranks_depth": rd[:N].copy(), "ranks_feat": rf[:N].copy(), "ranks_bev": rb[:N].copy(),
            "interval_starts": st[:I].copy(), "interval_lengths": ln[:I].copy(),
            "n_points": N, "n_intervals": I}


def forward(depth: np.ndarray, feat: np.ndarray, feat_dtype: str, feat_scale: float, C: int,
            m: dict, n_cells: int, with_abs: bool = False):
    """Scatter-reduce in double: returns out [n_cells, C] (and sum |terms| if with_abs).

    depth: float32/float16 array (any shape, read flat); feat: float32/float16
    array or uint8 e4m3 codes, read as [rows, C].
    """
    lib = _load()
    depth = np.ascontiguousarray(depth)
    feat = np.ascontiguousarray(feat)
    ddt = {np.dtype(np.float32): F32, np.dtype(np.float16): F16}[depth.dtype]
    fdt = _DTYPE_CODE[feat_dtype]
    expect = {F32: np.float32, F16: np.float16, E4M3: np.uint8}[fdt]
    if feat.dtype != expect:
        raise TypeError(f"feat dtype {feat.dtype} does not match {feat_dtype}")
    if feat.size % C:
        raise ValueError("feat size is not a multiple of C")
    rd = np.ascontiguousarray(m["ranks_depth"], np.int32)
    rf = np.ascontiguousarray(m["ranks_feat"], np.int32)
    rb = np.ascontiguousarray(m["ranks_bev"], np.int32)
    out = np.empty((n_cells, C), np.float64)
    out_abs = np.empty((n_cells, C), np.float64) if with_abs else None
    rc = lib.oracle_forward(_ptr(depth), ddt, depth.size, _ptr(feat), fdt, feat.size // C, C,
                            float(feat_scale), _ptr(rd), _ptr(rf), _ptr(rb), rd.size, n_cells,
                            _ptr(out), _ptr(out_abs) if with_abs else None)
    if rc != 0:
        raise ValueError(f"oracle_forward failed ({rc})")
    return (out, out_abs) if with_abs else out


def forward_threads(depth: np.ndarray, feat: np.ndarray, feat_dtype: str, feat_scale: float,
                    C: int, m: dict, n_cells: int, n_threads: int, with_abs: bool = False):
    """forward() spread over n_threads host threads, each taking a contiguous
    range of whole intervals of the map m (which must come from build_map:
    intervals tile the points, one per cell).  Bitwise equal to forward()."""
    lib = _load()
    depth = np.ascontiguousarray(depth)
    feat = np.ascontiguousarray(feat)
    ddt = {np.dtype(np.float32): F32, np.dtype(np.float16): F16}[depth.dtype]
    fdt = _DTYPE_CODE[feat_dtype]
    expect = {F32: np.float32, F16: np.float16, E4M3: np.uint8}[fdt]
    if feat.dtype != expect:
        raise TypeError(f"feat dtype {feat.dtype} does not match {feat_dtype}")
    arrs = {k: np.ascontiguousarray(m[k], np.int32)
            for k in ("ranks_depth", "ranks_feat", "ranks_bev", "interval_starts",
                      "interval_lengths")}
    out = np.empty((n_cells, C), np.float64)
    out_abs = np.empty((n_cells, C), np.float64) if with_abs else None
    rc = lib.oracle_forward_threads(
        _ptr(depth), ddt, depth.size, _ptr(feat), fdt, feat.size // C, C, float(feat_scale),
        _ptr(arrs["ranks_depth"]), _ptr(arrs["ranks_feat"]), _ptr(arrs["ranks_bev"]),
        arrs["ranks_bev"].size, _ptr(arrs["interval_starts"]), _ptr(arrs["interval_lengths"]),
        arrs["interval_starts"].size, n_cells, int(n_threads),
        _ptr(out), _ptr(out_abs) if with_abs else None)
    if rc != 0:
        raise ValueError(f"oracle_forward_threads failed ({rc})")
    return (out, out_abs) if with_abs else out


def segment_reduce(weights, table: np.ndarray, table_dtype: str, table_scale: float,
                   indices: np.ndarray, offsets: np.ndarray, with_abs: bool = False):
    """out[s] = sum_{t in [offsets[s], offsets[s+1])} w[t] * table[indices[t]] in double.

    weights: float32/float16 array [N] or None (all ones); table: [rows, C]
    float32/float16 or uint8 e4m3 codes.
    """
    lib = _load()
    table = np.ascontiguousarray(table)
    C = table.shape[-1]
    rows = table.size // C
    tdt = _DTYPE_CODE[table_dtype]
    expect = {F32: np.float32, F16: np.float16, E4M3: np.uint8}[tdt]
    if table.dtype != expect:
        raise TypeError(f"table dtype {table.dtype} does not match {table_dtype}")
    idx = np.ascontiguousarray(indices, np.int32)
    off = np.ascontiguousarray(offsets, np.int32)
    n_seg = off.size - 1
    wdt, wptr = 0, None
    if weights is not None:
        weights = np.ascontiguousarray(weights)
        wdt = {np.dtype(np.float32): F32, np.dtype(np.float16): F16}[weights.dtype]
        wptr = _ptr(weights)
    out = np.empty((n_seg, C), np.float64)
    out_abs = np.empty((n_seg, C), np.float64) if with_abs else None
    rc = lib.oracle_segment_reduce(wptr, wdt, _ptr(table), tdt, rows, C, float(table_scale),
                                   _ptr(idx), _ptr(off), n_seg, _ptr(out),
                                   _ptr(out_abs) if with_abs else None)
    if rc != 0:
        raise ValueError(f"oracle_segment_reduce failed ({rc})")
    return (out, out_abs) if with_abs else out
