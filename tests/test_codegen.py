"""Code-generation guards for the forward kernels (CPU: hipcc cross-compiles
gfx950, no GPU needed).

The measured speed of the pooling kernels rests on properties of the code
the compiler generates, not only on the source: a compiler update could undo
them silently.  This test compiles forward_kernels.hip to gfx950 assembly,
with the compiler's resource-usage remarks, and checks:
  * no kernel uses scratch memory (register spills go to scratch);
  * the kernels of the measured frames keep their occupancy: the C=80 fp16
    and e4m3 kernels, the C=128 and C=256 fp16 kernels and the C=128 fp16
    segment kernel at eight waves per SIMD (at most 64 VGPRs), the 16-byte
    e4m3 kernels (C=256, C=512) at six or more;
  * within a request round the row loads are not serialised: between two
    consecutive row loads on one path (no unconditional branch between them)
    there is never a wait for all outstanding vector memory operations
    (s_waitcnt vmcnt(0)) unless the round's accumulation (FMA instructions)
    lies between them -- the pattern of a compiler that cannot pair a load
    with its use across the round loop, which made every row load a separate
    round trip (20 % slower frames).  Checked to fire on such a build.
"""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "depth_weighted_scatter_amd", "csrc", "forward_kernels.hip")
HIPCC = "/opt/rocm/bin/hipcc"

# bev_pool_fwd<DT, FT, CB, G, SEG, OD> as mangled template arguments
# (DT/FT: 0 fp32, 1 fp16, 2 e4m3; CB: chunk bytes; G: chunks per row)
EIGHT_WAVES = {
    "fp16 C=80 (headline)": "Li1ELi1ELi16ELi10ELb0ELi0E",
    "e4m3 C=80": "Li1ELi2ELi8ELi10ELb0ELi0E",
    "fp16 C=128": "Li1ELi1ELi16ELi16ELb0ELi0E",
    "fp16 C=256": "Li1ELi1ELi16ELi32ELb0ELi0E",
    "fp16 C=128 segments": "Li1ELi1ELi16ELi16ELb1ELi0E",
}
SIX_WAVES = {
    "e4m3 C=256": "Li1ELi2ELi16ELi16ELb0ELi0E",
    "e4m3 C=512": "Li1ELi2ELi16ELi32ELb0ELi0E",
}
UNSERIALISED = dict(EIGHT_WAVES, **SIX_WAVES, **{
    "e4m3 C=128": "Li1ELi2ELi8ELi16ELb0ELi0E",
    "fp16 C=80 segments": "Li1ELi1ELi16ELi10ELb1ELi0E",
    "fp32 C=8 (tiny)": "Li0ELi0ELi16ELi2ELb0ELi0E",
})


def _mangled(args: str) -> str:
    return f"_ZN7bevpool12_GLOBAL__N_112bev_pool_fwdI{args}EEvNS_9FwdParamsE"


@pytest.fixture(scope="module")
def codegen(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("codegen") / "forward.s"
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
           f"-I{os.path.join(ROOT, 'include')}",
           f"-I{os.path.join(ROOT, 'depth_weighted_scatter_amd', 'csrc')}",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "--cuda-device-only", "-S", "-Rpass-analysis=kernel-resource-usage", SRC, "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, r.stderr[-3000:]
    usage, name = {}, None
    for line in r.stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            usage[name] = {}
            continue
        m = re.search(r"remark:\s+(VGPRs|ScratchSize \[bytes/lane\]|Occupancy \[waves/SIMD\]): (\d+)", line)
        if m and name:
            usage[name][m.group(1).split()[0]] = int(m.group(2))
    return out.read_text(), usage


def _body(asm: str, args: str):
    name = _mangled(args)
    i = asm.index(name + ":")
    j = asm.index(".Lfunc_end", i)
    return [ln.strip() for ln in asm[i:j].split("\n")
            if ln.startswith("\t") and not ln.strip().startswith((".", ";"))]


def test_no_kernel_uses_scratch(codegen):
    _, usage = codegen
    kernels = {k: v for k, v in usage.items() if "bev_pool_fwd" in k}
    assert len(kernels) > 300
    spilling = [k for k, v in kernels.items() if v.get("ScratchSize", 0) != 0]
    assert not spilling, f"kernels using scratch: {spilling[:5]}"


@pytest.mark.parametrize("label", list(EIGHT_WAVES))
def test_measured_kernels_keep_eight_waves(codegen, label):
    _, usage = codegen
    u = usage[_mangled(EIGHT_WAVES[label])]
    assert u["VGPRs"] <= 64 and u["Occupancy"] == 8, f"{label}: {u}"


@pytest.mark.parametrize("label", list(SIX_WAVES))
def test_e4m3_wide_kernels_keep_six_waves(codegen, label):
    _, usage = codegen
    u = usage[_mangled(SIX_WAVES[label])]
    assert u["Occupancy"] >= 6, f"{label}: {u}"


@pytest.mark.parametrize("label", list(UNSERIALISED))
def test_row_loads_within_a_round_are_not_serialised(codegen, label):
    asm, _ = codegen
    body = _body(asm, UNSERIALISED[label])
    loads = [i for i, ln in enumerate(body) if ln.startswith("buffer_load_dword")]
    assert loads, f"{label}: no row loads found"
    serial = []
    for a, b in zip(loads, loads[1:]):
        between = body[a + 1:b]
        if any(ln.startswith("s_branch") for ln in between):
            continue                      # textually adjacent, but on different paths
        if any("vmcnt(0)" in ln for ln in between) and not any(
                ln.startswith(("v_fma", "v_fmac")) for ln in between):
            serial.append(a)
    assert not serial, f"{label}: {len(serial)} row loads wait for every earlier load"
