"""bench.py's output contract: one JSON line with the metric, the roofline
object and the CPU-oracle baseline; more than one GPU is refused."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, BENCH, "--gpus", "2"], capture_output=True, text=True,
                       timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


@pytest.mark.gpu
def test_bench_prints_one_json_line():
    print("[bench contract] tiny workload", flush=True)
    r = subprocess.run([sys.executable, BENCH, "--workload", "0", "--steps", "100", "--warmup", "10",
                        "--cpu-seconds", "0.5"], capture_output=True, text=True, timeout=300,
                       cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, r.stdout
    d = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
              "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
              "roofline", "cpu_baseline"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 100 and d["warmup"] == 10
    assert d["value"] > 0 and d["ms_per_step"] > 0
    rf = d["roofline"]
    assert set(rf) >= {"bound", "achieved", "peak", "unit", "frac", "traffic"}
    assert rf["bound"] == "hbm" and rf["peak"] == 8000.0
    assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
    assert 0 < rf["compulsory_frac"] <= rf["frac"]
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["cores"] >= 1 and cb["value"] > 0 and cb["sample"]
    assert cb["single_core"]["cores"] == 1 and cb["hardware_concurrency"] >= cb["cores"]
    assert d["config"]["workload"] == "tiny"


def test_cpu_baseline_fields():
    """The CPU leg alone (no GPU needed): one-core and all-core oracle
    medians on the same workload, with the thread count it used."""
    sys.path.insert(0, ROOT)
    import bench
    import workloads
    wl = workloads.make_workload(0)
    s = wl.spec
    b_alg, _ = bench.algorithmic_bytes(s, int((wl.point_cell >= 0).sum()), 37)
    cb = bench.cpu_baseline(wl, b_alg, 1.0)
    assert cb["kind"] == "oracle" and cb["unit"] == "GB/s"
    assert cb["cores"] == bench.host_threads() >= 1
    assert cb["value"] > 0 and cb["single_core"]["value"] > 0 and cb["map_build_ms"] > 0
    assert cb["hardware_concurrency"] >= 1 and cb["cpu"]
