"""BEV pooling on MI355X (gfx950): Python binding of libbevpool.so.

The functions here carry the same names as the C ABI in include/bevpool.h
and only marshal arguments: PyTorch tensors supply device memory and the
current HIP stream, and every step of the computation runs in the library's
HIP kernels.  There is no CPU fallback -- if the library is missing or the
GPU is absent, calls raise.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional

import torch

__all__ = ["BevPoolError", "BevMap", "F32", "F16", "FP8_E4M3", "MAX_TABLE_BYTES", "library_path",
           "bevpool_status_string", "bevpool_version", "bevpool_build_map_workspace_size",
           "bevpool_build_map", "bevpool_build_map_no_alloc", "NO_ALLOC_MAP_SCRATCH_BYTES",
           "bevpool_forward", "bevpool_forward_baseline", "forward_args",
           "bevpool_forward_ex", "forward_ex_args", "BF16",
           "bevpool_segment_reduce", "segment_reduce_args",
           "ORDER_TILE_OUTER", "ORDER_DEPTH_OUTER"]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libbevpool.so")

F32, F16, FP8_E4M3, BF16 = 0, 1, 2, 3
# largest feature (or segment) table in bytes, BEVPOOL_MAX_TABLE_BYTES in bevpool.h
MAX_TABLE_BYTES = 2 ** 32 - 4096
# static device workspace of bevpool_build_map_no_alloc, BEVPOOL_NO_ALLOC_MAP_SCRATCH_BYTES
NO_ALLOC_MAP_SCRATCH_BYTES = 80 << 20
ORDER_TILE_OUTER, ORDER_DEPTH_OUTER = 0, 1
OK, ERR_CAPACITY = 0, -5

_TORCH_DTYPE_CODE = {torch.float32: F32, torch.float16: F16, torch.uint8: FP8_E4M3,
                     torch.float8_e4m3fn: FP8_E4M3}
_OUT_DTYPE_CODE = {torch.float32: F32, torch.float16: F16, torch.bfloat16: BF16}


class BevPoolError(RuntimeError):
    def __init__(self, func: str, status: int):
        super().__init__(f"{func} failed: {bevpool_status_string(status)} ({status})")
        self.status = status


_lib = None


def library_path() -> str:
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is not built; run __graft_entry__.build() "
                          "or python -m depth_weighted_scatter_amd.build")
    lib = ctypes.CDLL(_LIB_PATH)
    i32, i64, vp, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t
    lib.bevpool_status_string.restype = ctypes.c_char_p
    lib.bevpool_status_string.argtypes = [ctypes.c_int]
    lib.bevpool_version.restype = ctypes.c_int
    lib.bevpool_version.argtypes = []
    lib.bevpool_build_map_workspace_size.restype = sz
    lib.bevpool_build_map_workspace_size.argtypes = [i32, i32, i32, i32, i64]
    lib.bevpool_build_map.restype = ctypes.c_int
    lib.bevpool_build_map.argtypes = [vp, i32, i32, i32, i32, i64,
                                      vp, vp, vp, vp, vp, i64,
                                      ctypes.POINTER(i32), ctypes.POINTER(i32),
                                      vp, sz, vp]
    lib.bevpool_build_map_no_alloc.restype = ctypes.c_int
    lib.bevpool_build_map_no_alloc.argtypes = [vp, i32, i32, i32, i32, i64,
                                               vp, vp, vp, vp, vp, i64,
                                               ctypes.POINTER(i32), ctypes.POINTER(i32), vp]
    lib.bevpool_forward.restype = ctypes.c_int
    lib.bevpool_forward.argtypes = [vp, i32, i64, vp, i32, i64, i32, ctypes.c_float,
                                    vp, vp, vp, vp, vp, i32, i32, vp, i64, vp]
    lib.bevpool_forward_ex.restype = ctypes.c_int
    lib.bevpool_forward_ex.argtypes = [vp, i32, i64, vp, i32, i64, i32, ctypes.c_float,
                                       vp, vp, vp, vp, vp, i32, i32, vp, i32, i64, vp]
    lib.bevpool_forward_baseline.restype = ctypes.c_int
    lib.bevpool_forward_baseline.argtypes = [i32] + lib.bevpool_forward.argtypes
    lib.bevpool_segment_reduce.restype = ctypes.c_int
    lib.bevpool_segment_reduce.argtypes = [vp, i32, vp, i32, i64, i32, ctypes.c_float,
                                           vp, vp, i32, i32, vp, vp]
    _lib = lib
    return lib


def bevpool_status_string(status: int) -> str:
    return _load().bevpool_status_string(status).decode()


def bevpool_version() -> int:
    return _load().bevpool_version()


def bevpool_build_map_workspace_size(n_img: int, D: int, H: int, W: int, n_cells: int) -> int:
    return _load().bevpool_build_map_workspace_size(n_img, D, H, W, n_cells)


@dataclasses.dataclass
class BevMap:
    """The five INT32 scatter arrays (device tensors) and their counts."""
    ranks_depth: torch.Tensor
    ranks_feat: torch.Tensor
    ranks_bev: torch.Tensor
    interval_starts: torch.Tensor
    interval_lengths: torch.Tensor
    n_points: int
    n_intervals: int


def _stream_ptr(stream) -> Optional[int]:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _check_device_tensor(name, t, dtype=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def bevpool_build_map(point_cell: torch.Tensor, n_img: int, D: int, H: int, W: int,
                      n_cells: int, capacity: Optional[int] = None, stream=None) -> BevMap:
    """Five-array scatter map from point_cell (int32 [n_img*D*H*W], -1 = dropped).

    Allocates the map arrays (capacity entries each; default n_img*D*H*W) and
    the workspace with torch, then calls the library, which synchronises the
    stream once to read back the counts.
    """
    lib = _load()
    _check_device_tensor("point_cell", point_cell, torch.int32)
    P = n_img * D * H * W
    if point_cell.numel() != P:
        raise ValueError(f"point_cell has {point_cell.numel()} entries, expected {P}")
    cap = P if capacity is None else int(capacity)
    dev = point_cell.device
    ws_bytes = lib.bevpool_build_map_workspace_size(n_img, D, H, W, n_cells)
    if ws_bytes == 0:
        raise BevPoolError("bevpool_build_map_workspace_size", -1)
    ws = torch.empty(ws_bytes + 256, dtype=torch.uint8, device=dev)
    ws_ptr = (ws.data_ptr() + 255) & ~255
    arrs = [torch.empty(max(cap, 1), dtype=torch.int32, device=dev) for _ in range(5)]
    n_pts, n_iv = ctypes.c_int32(), ctypes.c_int32()
    rc = lib.bevpool_build_map(point_cell.data_ptr(), n_img, D, H, W, n_cells,
                               *(a.data_ptr() for a in arrs), cap,
                               ctypes.byref(n_pts), ctypes.byref(n_iv),
                               ws_ptr, ws_bytes, _stream_ptr(stream))
    if rc != OK:
        raise BevPoolError("bevpool_build_map", rc)
    N, I = n_pts.value, n_iv.value
    return BevMap(arrs[0][:N], arrs[1][:N], arrs[2][:N], arrs[3][:I], arrs[4][:I], N, I)


def bevpool_build_map_no_alloc(point_cell: torch.Tensor, n_img: int, D: int, H: int, W: int,
                               n_cells: int, arrays: Optional[list] = None,
                               stream=None) -> BevMap:
    """bevpool_build_map with the library's static device workspace: no
    workspace is allocated.  arrays: the five int32 output tensors
    (ranks_depth, ranks_feat, ranks_bev, interval_starts, interval_lengths),
    each of the same capacity; allocated here (n_img*D*H*W entries each) when
    None.  Calls on one device share the workspace: do not overlap them."""
    lib = _load()
    _check_device_tensor("point_cell", point_cell, torch.int32)
    P = n_img * D * H * W
    if point_cell.numel() != P:
        raise ValueError(f"point_cell has {point_cell.numel()} entries, expected {P}")
    if arrays is None:
        arrays = [torch.empty(max(P, 1), dtype=torch.int32, device=point_cell.device)
                  for _ in range(5)]
    if len(arrays) != 5:
        raise ValueError("arrays must hold the five map arrays")
    for a in arrays:
        _check_device_tensor("map array", a, torch.int32)
    cap = min(a.numel() for a in arrays)
    n_pts, n_iv = ctypes.c_int32(), ctypes.c_int32()
    rc = lib.bevpool_build_map_no_alloc(point_cell.data_ptr(), n_img, D, H, W, n_cells,
                                        *(a.data_ptr() for a in arrays), cap,
                                        ctypes.byref(n_pts), ctypes.byref(n_iv),
                                        _stream_ptr(stream))
    if rc != OK:
        raise BevPoolError("bevpool_build_map_no_alloc", rc)
    N, I = n_pts.value, n_iv.value
    return BevMap(arrays[0][:N], arrays[1][:N], arrays[2][:N], arrays[3][:I], arrays[4][:I], N, I)


def _forward_inputs(depth: torch.Tensor, feat: torch.Tensor, m: BevMap, n_cells: int,
                    out: torch.Tensor, feat_scale: float) -> tuple:
    # Checks shared by the forward entry points; returns the C arguments up
    # to n_intervals (out, its type, n_cells and the stream follow).
    _check_device_tensor("depth", depth)
    _check_device_tensor("feat", feat)
    _check_device_tensor("out", out)
    for name in ("ranks_depth", "ranks_feat", "ranks_bev"):
        _check_device_tensor(name, getattr(m, name), torch.int32)
        if getattr(m, name).numel() < m.n_points:
            raise ValueError(f"{name} holds fewer than n_points = {m.n_points} entries")
    for name in ("interval_starts", "interval_lengths"):
        _check_device_tensor(name, getattr(m, name), torch.int32)
        if getattr(m, name).numel() < m.n_intervals:
            raise ValueError(f"{name} holds fewer than n_intervals = {m.n_intervals} entries")
    if depth.dtype not in (torch.float32, torch.float16):
        raise TypeError(f"depth must be float32 or float16, got {depth.dtype}")
    if feat.dtype not in _TORCH_DTYPE_CODE:
        raise TypeError(f"feat dtype {feat.dtype} is not supported")
    C = feat.shape[-1]
    if out.numel() != n_cells * C:
        raise ValueError(f"out has {out.numel()} elements, expected {n_cells}*{C}")
    return (depth.data_ptr(), _TORCH_DTYPE_CODE[depth.dtype], depth.numel(),
            feat.data_ptr(), _TORCH_DTYPE_CODE[feat.dtype], feat.numel() // C, C,
            float(feat_scale),
            m.ranks_depth.data_ptr(), m.ranks_feat.data_ptr(), m.ranks_bev.data_ptr(),
            m.interval_starts.data_ptr(), m.interval_lengths.data_ptr(),
            m.n_points, m.n_intervals)


def forward_args(depth: torch.Tensor, feat: torch.Tensor, m: BevMap, n_cells: int,
                 out: torch.Tensor, feat_scale: float = 1.0, stream=None) -> tuple:
    """Validated, marshalled argument tuple for the C bevpool_forward.

    Lets a caller that launches many times (a benchmark, a graph capture)
    pay the Python-side checks once: _load().bevpool_forward(*args).
    """
    _check_device_tensor("out", out, torch.float32)
    return _forward_inputs(depth, feat, m, n_cells, out, feat_scale) + (
        out.data_ptr(), n_cells, _stream_ptr(stream))


def forward_ex_args(depth: torch.Tensor, feat: torch.Tensor, m: BevMap, n_cells: int,
                    out: torch.Tensor, feat_scale: float = 1.0, stream=None) -> tuple:
    """Marshalled argument tuple for the C bevpool_forward_ex; the output
    type (float32, float16 or bfloat16) is out's dtype."""
    if out.dtype not in _OUT_DTYPE_CODE:
        raise TypeError(f"out must be float32, float16 or bfloat16, got {out.dtype}")
    return _forward_inputs(depth, feat, m, n_cells, out, feat_scale) + (
        out.data_ptr(), _OUT_DTYPE_CODE[out.dtype], n_cells, _stream_ptr(stream))


def bevpool_forward(depth: torch.Tensor, feat: torch.Tensor, m: BevMap, n_cells: int,
                    feat_scale: float = 1.0, out: Optional[torch.Tensor] = None,
                    stream=None) -> torch.Tensor:
    """Depth-weighted interval-owned scatter-reduce; returns out [n_cells, C] fp32.

    depth: float32 / float16 (any shape, read flat); feat: [..., C] float32,
    float16, or OCP e4m3 (torch.float8_e4m3fn or its uint8 codes) with
    feat_scale.  Enqueued on the current stream; never synchronises.
    """
    lib = _load()
    if out is None:
        out = torch.empty((n_cells, feat.shape[-1]), dtype=torch.float32, device=feat.device)
    rc = lib.bevpool_forward(*forward_args(depth, feat, m, n_cells, out, feat_scale, stream))
    if rc != OK:
        raise BevPoolError("bevpool_forward", rc)
    return out


def bevpool_forward_ex(depth: torch.Tensor, feat: torch.Tensor, m: BevMap, n_cells: int,
                       out_dtype: torch.dtype = torch.float16, feat_scale: float = 1.0,
                       out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """bevpool_forward with the fp32 sums rounded (nearest-even) to out_dtype
    (float32, float16 or bfloat16) at the store; returns out [n_cells, C]."""
    lib = _load()
    if out is None:
        out = torch.empty((n_cells, feat.shape[-1]), dtype=out_dtype, device=feat.device)
    rc = lib.bevpool_forward_ex(*forward_ex_args(depth, feat, m, n_cells, out, feat_scale,
                                                 stream))
    if rc != OK:
        raise BevPoolError("bevpool_forward_ex", rc)
    return out


def bevpool_forward_baseline(order: int, depth: torch.Tensor, feat: torch.Tensor, m: BevMap,
                             n_cells: int, feat_scale: float = 1.0,
                             out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """The article's earlier loop orders (ORDER_TILE_OUTER = V2-style,
    ORDER_DEPTH_OUTER = V2+DO-style) with bevpool_forward's arguments and
    results; a comparison baseline, not a fast path."""
    lib = _load()
    if out is None:
        out = torch.empty((n_cells, feat.shape[-1]), dtype=torch.float32, device=feat.device)
    rc = lib.bevpool_forward_baseline(order, *forward_args(depth, feat, m, n_cells, out,
                                                           feat_scale, stream))
    if rc != OK:
        raise BevPoolError("bevpool_forward_baseline", rc)
    return out


def segment_reduce_args(weights: Optional[torch.Tensor], table: torch.Tensor,
                        indices: torch.Tensor, offsets: torch.Tensor, out: torch.Tensor,
                        table_scale: float = 1.0, stream=None) -> tuple:
    """Validated, marshalled argument tuple for the C bevpool_segment_reduce."""
    _check_device_tensor("table", table)
    _check_device_tensor("indices", indices, torch.int32)
    _check_device_tensor("offsets", offsets, torch.int32)
    _check_device_tensor("out", out, torch.float32)
    if table.dtype not in _TORCH_DTYPE_CODE:
        raise TypeError(f"table dtype {table.dtype} is not supported")
    C = table.shape[-1]
    n_seg = offsets.numel() - 1
    if n_seg < 0 or out.numel() != n_seg * C:
        raise ValueError("out must be [len(offsets) - 1, C]")
    if weights is not None:
        _check_device_tensor("weights", weights)
        if weights.dtype not in (torch.float32, torch.float16):
            raise TypeError(f"weights must be float32 or float16, got {weights.dtype}")
        if weights.numel() != indices.numel():
            raise ValueError("weights and indices differ in length")
        wdt, wptr = _TORCH_DTYPE_CODE[weights.dtype], weights.data_ptr()
    else:
        wdt, wptr = (F32 if table.dtype == torch.float32 else F16), None
    return (wptr, wdt, table.data_ptr(), _TORCH_DTYPE_CODE[table.dtype], table.numel() // C, C,
            float(table_scale), indices.data_ptr(), offsets.data_ptr(), n_seg, indices.numel(),
            out.data_ptr(), _stream_ptr(stream))


def bevpool_segment_reduce(weights: Optional[torch.Tensor], table: torch.Tensor,
                           indices: torch.Tensor, offsets: torch.Tensor,
                           table_scale: float = 1.0, out: Optional[torch.Tensor] = None,
                           stream=None) -> torch.Tensor:
    """out[s] = sum_{t in [offsets[s], offsets[s+1])} weights[t] * table[indices[t]]
    (weights None = 1); fp32 [len(offsets) - 1, C].  Enqueued on the current
    stream; never synchronises."""
    lib = _load()
    if out is None:
        out = torch.empty((offsets.numel() - 1, table.shape[-1]), dtype=torch.float32,
                          device=table.device)
    rc = lib.bevpool_segment_reduce(*segment_reduce_args(weights, table, indices, offsets, out,
                                                         table_scale, stream))
    if rc != OK:
        raise BevPoolError("bevpool_segment_reduce", rc)
    return out
