"""Host-side validation of the C ABI with real device buffers.

The CPU suite (test_abi.py) checks every rejection with device pointers that
map nothing, which is safe only where no GPU is visible.  Here bad arguments
are passed with small real allocations and a valid two-interval map, and
only kinds of bad argument whose kernel would still stay inside these
buffers if validation were ever skipped (misalignment, an unsupported type
pair or width, a short or misaligned workspace); the size-overflow cases stay
CPU-only.  Each call must return its status without touching the output,
which holds a sentinel that is compared afterwards.
"""
import ctypes

import pytest
import torch

import depth_weighted_scatter_amd as dws
from gpu_util import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bufs():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    dev = torch.device("cuda:0")

    def i32(v):
        return torch.tensor(v + [0] * (64 - len(v)), dtype=torch.int32, device=dev)

    b = {"depth": torch.ones(64, dtype=torch.float16, device=dev),
         "feat": torch.ones(4096, dtype=torch.float16, device=dev),
         # a valid map: 5 points in cells 0 and 1 (intervals of 3 and 2 points)
         "rd": i32([0, 1, 2, 3, 4]), "rf": i32([0, 1, 2, 3, 4]), "rb": i32([0, 0, 0, 1, 1]),
         "st": i32([0, 3]), "ln": i32([3, 2]),
         "pc": i32([0, 1, 2, 3, 0, 1, 2, 3]), "ws": torch.zeros(1 << 16, dtype=torch.uint8, device=dev),
         "out": torch.full((4096,), 7.0, dtype=torch.float32, device=dev)}
    torch.cuda.synchronize()
    return b


def _fwd_args(b, **kw):
    a = dict(depth=b["depth"].data_ptr(), ddt=dws.F16, n_depth=64, feat=b["feat"].data_ptr(),
             fdt=dws.F16, rows=10, C=80, scale=1.0, rd=b["rd"].data_ptr(), rf=b["rf"].data_ptr(),
             rb=b["rb"].data_ptr(), st=b["st"].data_ptr(), ln=b["ln"].data_ptr(), n_points=5,
             n_iv=2)
    a.update(kw)
    return list(a.values())


@pytest.mark.parametrize("case,kw,code", [
    ("f32 depth with f16 features", dict(ddt=dws.F32), -2),
    ("24-byte rows", dict(C=12), -2),
    ("misaligned output", "out+4", -1),
    ("misaligned features", dict(feat="feat+8"), -1),
])
def test_forward_rejects_with_real_buffers(bufs, case, kw, code):
    lib = dws._load()
    s = torch.cuda.current_stream().cuda_stream
    out = bufs["out"].data_ptr()
    if kw == "out+4":
        kw, out = {}, out + 4
    if kw.get("feat") == "feat+8":
        kw = dict(feat=bufs["feat"].data_ptr() + 8)
    say(f"[abi errors, real buffers] forward: {case}")
    assert lib.bevpool_forward(*_fwd_args(bufs, **kw), out, 16, s) == code
    assert lib.bevpool_forward_ex(*_fwd_args(bufs, **kw), out, dws.F32, 16, s) == code
    assert lib.bevpool_forward_baseline(1, *_fwd_args(bufs, **kw), out, 16, s) == code
    torch.cuda.synchronize()
    assert (bufs["out"] == 7.0).all(), "a rejected call wrote the output"


def test_segment_reduce_and_map_reject_with_real_buffers(bufs):
    lib = dws._load()
    s = torch.cuda.current_stream().cuda_stream
    p = {k: v.data_ptr() for k, v in bufs.items()}
    say("[abi errors, real buffers] segment reduce and map build")
    # offsets = interval starts [0, 3] then zeros: segment 0 holds 3 points
    assert lib.bevpool_segment_reduce(p["depth"], dws.F32, p["feat"], dws.F16, 10, 80, 1.0,
                                      p["rf"], p["st"], 1, 5, p["out"], s) == -2
    assert lib.bevpool_segment_reduce(p["depth"], dws.F16, p["feat"], dws.F16, 10, 80, 1.0,
                                      p["rf"], p["st"], 1, 5, p["out"] + 4, s) == -1
    assert lib.bevpool_segment_reduce(None, dws.F16, p["feat"], dws.F16, 10, 12, 1.0,
                                      p["rf"], p["st"], 1, 5, p["out"], s) == -2
    n_pts, n_iv = ctypes.c_int32(), ctypes.c_int32()
    need = lib.bevpool_build_map_workspace_size(1, 2, 2, 2, 4)
    assert 0 < need <= (1 << 16) - 256
    args = [p["pc"], 1, 2, 2, 2, 4, p["rd"], p["rf"], p["rb"], p["st"], p["ln"], 8,
            ctypes.byref(n_pts), ctypes.byref(n_iv)]
    assert lib.bevpool_build_map(*args, p["ws"], need - 1, s) == -4       # workspace short
    assert lib.bevpool_build_map(*args, p["ws"] + 64, need, s) == -4      # not 256-byte aligned
    torch.cuda.synchronize()
    assert (bufs["out"] == 7.0).all(), "a rejected call wrote the output"
    # the map arrays were not touched either
    assert bufs["rb"][:5].tolist() == [0, 0, 0, 1, 1] and bufs["ln"][:2].tolist() == [3, 2]


def test_binding_rejects_bad_map_tensors(bufs):
    """The Python binding checks the map's tensors before anything reaches the
    library: a host tensor, a wrong dtype or an array shorter than its count
    raises, and the output keeps its sentinel."""
    import dataclasses
    b = bufs
    m = dws.BevMap(b["rd"], b["rf"], b["rb"], b["st"], b["ln"], 5, 2)
    depth, feat = b["depth"], b["feat"][:800].view(10, 80)
    out = torch.full((16, 80), 7.0, dtype=torch.float32, device=depth.device)
    bad = [(TypeError, dataclasses.replace(m, ranks_feat=b["rf"].cpu())),
           (TypeError, dataclasses.replace(m, ranks_bev=b["rb"].to(torch.int64))),
           (ValueError, dataclasses.replace(m, ranks_depth=b["rd"][:4])),
           (ValueError, dataclasses.replace(m, interval_lengths=b["ln"][:1]))]
    for err, mm in bad:
        with pytest.raises(err):
            dws.bevpool_forward(depth, feat, mm, 16, out=out)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all()), "a rejected call wrote the output"
    with pytest.raises(TypeError):
        dws.bevpool_segment_reduce(b["depth"][:5].to(torch.bfloat16), feat, b["rf"][:5],
                                   b["st"][:2], out=out[:1])
