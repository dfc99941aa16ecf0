"""C ABI checks that need no GPU: the library loads, exports every function
include/bevpool.h declares, and rejects bad arguments on the host before any
HIP call (no kernel is launched here)."""
import ctypes
import os
import re

import pytest

import depth_weighted_scatter_amd as dws


def _gpu_visible() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bevpool.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bevpool_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(dws.library_path()):
        import depth_weighted_scatter_amd.build as b
        b.build()
    return dws._load()


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("bevpool_build_map", "bevpool_forward", "bevpool_build_map_workspace_size",
                     "bevpool_status_string"):
        assert required in names


def test_table_limit_matches_header():
    with open(os.path.join(os.path.dirname(dws.library_path()), "..", "include", "bevpool.h")) as f:
        m = re.search(r"#define BEVPOOL_MAX_TABLE_BYTES (\d+)u", f.read())
    assert m and int(m.group(1)) == dws.MAX_TABLE_BYTES == 2 ** 32 - 4096


def test_every_declared_symbol_is_exported(lib):
    handle = ctypes.CDLL(dws.library_path())
    for name in declared_functions():
        assert hasattr(handle, name), f"{name} declared in bevpool.h but not exported"


def test_status_strings(lib):
    for code in range(0, -8, -1):
        s = dws.bevpool_status_string(code)
        assert s and s != "unknown status"
    assert dws.bevpool_status_string(-99) == "unknown status"
    assert dws.bevpool_version() >= 10000


def test_workspace_size(lib):
    assert dws.bevpool_build_map_workspace_size(6, 59, 16, 44, 128 * 128) > 5 * 249216 * 4
    assert dws.bevpool_build_map_workspace_size(0, 1, 1, 1, 10) == 0
    assert dws.bevpool_build_map_workspace_size(1, 1, 1, 1, 0) == 0
    assert dws.bevpool_build_map_workspace_size(1 << 15, 1 << 15, 4, 1, 10) == 0  # P >= 2^31
    # a frustum whose int64 product n_img*D*H*W would wrap (2^120 -> 0) is still too large
    assert dws.bevpool_build_map_workspace_size(1 << 30, 1 << 30, 1 << 30, 1 << 30, 10) == 0
    assert dws.bevpool_build_map_workspace_size(2**31 - 1, 2**31 - 1, 2**31 - 1, 2**31 - 1, 10) == 0


FAKE = 1 << 40          # never dereferenced: validation fails first

# The rejection tests below hand the real entry points device pointers that
# map nothing.  With a GPU visible, a regression in host validation would
# launch a kernel at that address, so they run only where no GPU is visible
# (the GPU suite checks argument errors with real buffers instead).
no_gpu_only = pytest.mark.skipif(_gpu_visible(), reason="fake device pointers: CPU-only check")


def _fwd(lib, **kw):
    a = dict(depth=FAKE, ddt=dws.F16, n_depth=100, feat=FAKE, fdt=dws.F16, rows=10, C=80,
             scale=1.0, rd=FAKE, rf=FAKE, rb=FAKE, st=FAKE, ln=FAKE, n_points=5, n_iv=2,
             out=FAKE, n_cells=16, stream=None)
    a.update(kw)
    return lib.bevpool_forward(*a.values())


@no_gpu_only
@pytest.mark.parametrize("kw,code", [
    (dict(out=None), -1),
    (dict(depth=None), -1),
    (dict(rd=None), -1),
    (dict(C=0), -1),
    (dict(n_cells=0), -1),
    (dict(n_iv=6), -1),                         # more intervals than points
    (dict(n_points=-1), -1),
    (dict(ddt=dws.F32), -2),                    # f32 depth with f16 feat
    (dict(fdt=7), -2),
    (dict(C=12), -2),                           # 24-byte rows are not 16-byte chunks
    (dict(C=1024), -2),                         # 2 KB rows
    (dict(fdt=dws.FP8_E4M3, C=4), -2),          # 4-byte fp8 rows
    (dict(fdt=dws.FP8_E4M3, C=520), -2),        # fp8 rows over 512 bytes must be 16-byte multiples
    (dict(fdt=dws.FP8_E4M3, C=2048), -2),
    (dict(n_cells=1 << 26, C=64), -3),          # n_cells * C >= 2^31
    (dict(rows=1 << 26, C=64), -3),
    (dict(ddt=dws.F32, fdt=dws.F32, rows=(1 << 24) + 1, C=64), -3),   # fp32 table of 4 GiB + 256 B
    (dict(ddt=dws.F32, fdt=dws.F32, rows=16777201, C=64), -3),        # 256 B over the table limit
    (dict(rows=8388601, C=256), -3),            # fp16 table 512 B over the limit, rows*C < 2^31
    (dict(n_cells=1 << 62, C=8), -3),           # n_cells * C would wrap to 0 in int64
    (dict(rows=1 << 62, C=64), -3),             # rows * row bytes would wrap to 0
    (dict(n_depth=1 << 62), -3),
    (dict(out=FAKE + 4), -1),                   # misaligned output
    (dict(feat=FAKE + 8), -1),                  # misaligned features
])
def test_forward_rejects(lib, kw, code):
    assert _fwd(lib, **kw) == code


def _fwd_ex(lib, **kw):
    a = dict(depth=FAKE, ddt=dws.F16, n_depth=100, feat=FAKE, fdt=dws.F16, rows=10, C=80,
             scale=1.0, rd=FAKE, rf=FAKE, rb=FAKE, st=FAKE, ln=FAKE, n_points=5, n_iv=2,
             out=FAKE, odt=dws.F16, n_cells=16, stream=None)
    a.update(kw)
    return lib.bevpool_forward_ex(*a.values())


@no_gpu_only
@pytest.mark.parametrize("kw,code", [
    (dict(odt=dws.FP8_E4M3), -2),               # e4m3 is not an output type
    (dict(odt=4), -2),
    (dict(odt=-1), -2),
    (dict(out=None), -1),
    (dict(out=FAKE + 4), -1),                   # 16-bit output must be 8-byte aligned
    (dict(odt=dws.BF16, out=FAKE + 2), -1),
    (dict(odt=dws.F32, out=FAKE + 8), -1),      # fp32 output must be 16-byte aligned
    (dict(ddt=dws.F32), -2),                    # input checks are bevpool_forward's
    (dict(C=12), -2),
    (dict(n_cells=1 << 26, C=64), -3),
])
def test_forward_ex_rejects(lib, kw, code):
    assert _fwd_ex(lib, **kw) == code


def _map(lib, **kw):
    n_pts, n_iv = ctypes.c_int32(), ctypes.c_int32()
    a = dict(pc=FAKE, n_img=1, D=2, H=2, W=2, n_cells=4, rd=FAKE, rf=FAKE, rb=FAKE, st=FAKE,
             ln=FAKE, cap=8, hn=ctypes.byref(n_pts), hi=ctypes.byref(n_iv), ws=FAKE,
             ws_bytes=1 << 20, stream=None)
    a.update(kw)
    return lib.bevpool_build_map(*a.values())


@no_gpu_only
@pytest.mark.parametrize("kw,code", [
    (dict(pc=None), -1),
    (dict(ln=None), -1),
    (dict(ws=None), -1),
    (dict(D=0), -1),
    (dict(n_cells=0), -1),
    (dict(cap=-1), -1),
    (dict(n_img=1 << 16, D=1 << 16), -3),        # P >= 2^31
    (dict(n_img=1 << 30, D=1 << 30, H=1 << 30, W=1 << 30), -3),   # the int64 product would wrap to 0
    (dict(n_cells=1 << 31), -3),
    (dict(ws_bytes=16), -4),
    (dict(ws=FAKE + 64), -4),                    # workspace not 256-byte aligned
])
def test_build_map_rejects(lib, kw, code):
    assert _map(lib, **kw) == code


def _map_no_alloc(lib, **kw):
    n_pts, n_iv = ctypes.c_int32(), ctypes.c_int32()
    a = dict(pc=FAKE, n_img=1, D=2, H=2, W=2, n_cells=4, rd=FAKE, rf=FAKE, rb=FAKE, st=FAKE,
             ln=FAKE, cap=8, hn=ctypes.byref(n_pts), hi=ctypes.byref(n_iv), stream=None)
    a.update(kw)
    return lib.bevpool_build_map_no_alloc(*a.values())


@no_gpu_only
@pytest.mark.parametrize("kw,code", [
    (dict(n_img=96, D=59, H=32, W=88), -4),      # 15.9 M points: past the 80 MiB workspace
    (dict(n_img=1, D=1, H=1, W=4091521), -4),    # one point past the largest frustum
    (dict(pc=None), -1),
    (dict(ln=None), -1),
    (dict(D=0), -1),
    (dict(cap=-1), -1),
    (dict(n_img=1 << 16, D=1 << 16), -3),        # P >= 2^31
    (dict(n_img=1 << 30, D=1 << 30, H=1 << 30, W=1 << 30), -3),   # the int64 product would wrap to 0
    (dict(n_cells=1 << 31), -3),
])
def test_build_map_no_alloc_rejects(lib, kw, code):
    assert _map_no_alloc(lib, **kw) == code


def test_no_alloc_limit_matches_header(lib):
    with open(HEADER) as f:
        m = re.search(r"#define BEVPOOL_NO_ALLOC_MAP_SCRATCH_BYTES \((\d+)u << (\d+)\)", f.read())
    assert m and int(m.group(1)) << int(m.group(2)) == dws.NO_ALLOC_MAP_SCRATCH_BYTES
    # the largest frustum the header names fits, one more point does not
    assert dws.bevpool_build_map_workspace_size(1, 1, 1, 4091520, 4) <= dws.NO_ALLOC_MAP_SCRATCH_BYTES
    assert dws.bevpool_build_map_workspace_size(1, 1, 1, 4091521, 4) > dws.NO_ALLOC_MAP_SCRATCH_BYTES


@no_gpu_only
def test_baseline_rejects(lib):
    a = dict(depth=FAKE, ddt=dws.F16, n_depth=100, feat=FAKE, fdt=dws.F16, rows=10, C=80,
             scale=1.0, rd=FAKE, rf=FAKE, rb=FAKE, st=FAKE, ln=FAKE, n_points=5, n_iv=2,
             out=FAKE, n_cells=16, stream=None)
    assert lib.bevpool_forward_baseline(7, *a.values()) == -1          # unknown order
    b = dict(a, fdt=dws.FP8_E4M3, C=40)                                  # 40-byte rows
    assert lib.bevpool_forward_baseline(0, *b.values()) == -2
    assert lib.bevpool_forward_baseline(1, *dict(a, out=None).values()) == -1


@no_gpu_only
@pytest.mark.parametrize("kw,code", [
    (dict(table=None), -1),
    (dict(idx=None), -1),
    (dict(off=None), -1),
    (dict(out=None), -1),
    (dict(n_seg=-1), -1),
    (dict(C=0), -1),
    (dict(tdt=dws.F16, wdt=dws.F32), -2),
    (dict(C=12), -2),
    (dict(n_seg=1 << 26, C=64), -3),
    (dict(wdt=dws.F32, tdt=dws.F32, rows=1 << 24, C=64), -3),          # fp32 table of 4 GiB
    (dict(wdt=dws.F32, tdt=dws.F32, rows=16777201, C=64), -3),         # 256 B over the table limit
    (dict(rows=1 << 62, C=64), -3),                                    # rows * row bytes would wrap to 0
    (dict(out=FAKE + 4), -1),
])
def test_segment_reduce_rejects(lib, kw, code):
    a = dict(w=FAKE, wdt=dws.F16, table=FAKE, tdt=dws.F16, rows=10, C=80, scale=1.0, idx=FAKE,
             off=FAKE, n_seg=4, n_pts=20, out=FAKE, stream=None)
    a.update(kw)
    assert lib.bevpool_segment_reduce(*a.values()) == code


def test_segment_reduce_empty_is_noop(lib):
    assert lib.bevpool_segment_reduce(None, 1, None, 1, 0, 8, 1.0, None, None, 0, 0, None, None) == 0
