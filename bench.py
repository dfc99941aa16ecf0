"""Benchmark of bevpool_forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 1]

One step is one bevpool_forward call: the whole pooled forward (interval
headers, index and depth reads, feature-row gathers, fp32 accumulation,
owned-row and empty-cell stores) over one frame of synthetic input.  The
scatter map is built once beforehand (it is prepared once per geometry; its
build time is reported separately).  Inputs are resident in HBM before
timing starts.  The K timed steps run as HIP-graph replays of back-to-back
forward calls on one stream, bracketed by device synchronisation and timed
with HIP events on that stream.

Prints ONE JSON line.  value = effective bandwidth in GB/s of the
algorithmic bytes
    B_alg = N*(C*e_feat + e_depth + 12) + 8*I + n_cells*C*4
(one feature row, one depth value and three INT32 indices per scatter point,
two INT32 per interval, one fp32 write per output element) per call time.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "bevpool_forward µs/call + effective GB/s (% HBM peak), 6cam×59D×16×44, C=80"
KERNEL_SRC = os.path.join(ROOT, "depth_weighted_scatter_amd", "csrc", "forward_kernels.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
ELEM_BYTES = {"f32": 4, "f16": 2, "e4m3": 1}


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", type=int, default=1, help="synthetic workload 0..4 (1 = headline)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--graph-chunk", type=int, default=50, help="forward calls per captured graph")
    ap.add_argument("--eager", action="store_true", help="time eager launches instead of graph replay")
    ap.add_argument("--bags", type=int, default=None,
                    help="benchmark bevpool_segment_reduce on embedding-bag workload k instead")
    ap.add_argument("--kernel", choices=["owned", "v2", "v2do"], default="owned",
                    help="owned: bevpool_forward; v2 / v2do: the tile-outer / depth-outer baselines")
    ap.add_argument("--out-dtype", choices=["f32", "f16", "bf16"], default="f32",
                    help="output type of the owned kernel (f16/bf16 via bevpool_forward_ex)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="CPU-oracle sample length")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--copy-calib-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (counter calibration)")
    ap.add_argument("--details", default=None, help="write extra measurements as JSON here")
    ap.add_argument("--summarize", nargs=4, metavar=("TRACE_DIR", "FETCH_DIR", "WRITE_DIR", "BENCH_JSON"),
                    default=None,
                    help="(CPU) turn rocprofv3 csv output of this benchmark into a summary under "
                         "profiles/ and update profiles/traffic.json, then exit")
    ap.add_argument("--commands", default="", help="with --summarize: the commands that made the inputs")
    ap.add_argument("--pmc-dirs", nargs="*", default=[],
                    help="with --summarize: further rocprofv3 --pmc output directories whose "
                         "counters for the forward kernel are listed (L2 hit rate from "
                         "TCC_HIT_sum / TCC_MISS_sum when present)")
    return ap.parse_args()


def algorithmic_bytes(spec, N, I, out_bytes=4):
    per_point = spec.C * ELEM_BYTES[spec.feat_dtype] + ELEM_BYTES[spec.depth_dtype] + 12
    b_alg = N * per_point + 8 * I + spec.n_cells * spec.C * out_bytes
    b_min = (spec.n_feat_rows * spec.C * ELEM_BYTES[spec.feat_dtype]
             + spec.n_img * spec.D * spec.H * spec.W * ELEM_BYTES[spec.depth_dtype]
             + 12 * N + 8 * I + spec.n_cells * spec.C * out_bytes)
    return b_alg, b_min


def kernel_hash() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def traffic_for(workload_name: str):
    """HBM bytes per launch from committed rocprofv3 counters, if they were
    taken on the current kernel source; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    ent = rec.get(workload_name)
    if not ent or ent.get("kernel_sha256_16") != kernel_hash():
        return None
    return ent.get("hbm_bytes_per_launch")


def _read_csv(directory, suffix):
    import csv
    import glob
    paths = sorted(glob.glob(os.path.join(directory, "**", f"*{suffix}"), recursive=True))
    if not paths:
        raise FileNotFoundError(f"no *{suffix} under {directory}")
    with open(paths[0]) as f:
        return list(csv.DictReader(f))


def _counter_means(directory, counter):
    """Mean counter value per dispatch, by kernel name (rocprofv3 --pmc csv)."""
    sums, counts = {}, {}
    for r in _read_csv(directory, "counter_collection.csv"):
        if r["Counter_Name"] != counter:
            continue
        k = r["Kernel_Name"]
        sums[k] = sums.get(k, 0.0) + float(r["Counter_Value"])
        counts[k] = counts.get(k, 0) + 1
    return {k: sums[k] / counts[k] for k in sums}


def summarize(args):
    """Write profiles/<kernel>_<workload>.md and update profiles/traffic.json."""
    trace_dir, fetch_dir, write_dir, bench_json = args.summarize
    with open(bench_json) as f:
        bench = json.loads(f.read().strip().splitlines()[-1])
    workload = bench["config"]["workload"]
    stats = _read_csv(trace_dir, "kernel_stats.csv")
    fwd = [r for r in stats if "bev_pool_fwd" in r["Name"]]
    fetch = _counter_means(fetch_dir, "FETCH_SIZE")
    write = _counter_means(write_dir, "WRITE_SIZE")

    def pick(d, key):
        return next((v for k, v in d.items() if key in k), None)

    fwd_fetch, fwd_write = pick(fetch, "bev_pool_fwd"), pick(write, "bev_pool_fwd")
    copy_fetch = pick(fetch, "bitwise_not")   # the calibration copy: reads and writes copy_kib
    copy_write = pick(write, "bitwise_not")
    copy_kib = bench.get("secondary", {}).get("copy_calib_mib", 0) * 1024
    f_scale = copy_kib / copy_fetch if copy_fetch and copy_kib else None
    w_scale = copy_kib / copy_write if copy_write and copy_kib else None
    traffic = None
    if fwd_fetch is not None and fwd_write is not None and f_scale and w_scale:
        traffic = int(round((fwd_fetch * f_scale + fwd_write * w_scale) * 1024))
    avg_ns = float(fwd[0]["AverageNs"]) if fwd else None
    # per-dispatch durations of the forward kernel from the same trace
    durs = sorted(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
                  for r in _read_csv(trace_dir, "kernel_trace.csv") if "bev_pool_fwd" in r["Kernel_Name"])
    med_ns = durs[len(durs) // 2] if durs else None
    p10_ns = durs[len(durs) // 10] if durs else None
    name = "bev_pool_fwd"
    lines = [f"# {name} on {workload} (MI355X, gfx950)", "",
             "Commands (from the repository root):", "", "```", args.commands.strip(), "```", "",
             "## Kernel trace (rocprofv3 --kernel-trace --stats)", "",
             "| kernel | calls | average ns | min ns | max ns |", "|---|---|---|---|---|"]
    for r in stats[:8]:
        lines.append(f"| {r['Name'][:90]} | {r['Calls']} | {float(r['AverageNs']):.0f} | "
                     f"{r['MinNs']} | {r['MaxNs']} |")
    lines += ["", "## Benchmark line (same build)", "",
              f"- per call (HIP events, graph replay): {bench['us_per_call']} us",
              f"- rocprof average kernel duration: {avg_ns / 1e3:.3f} us" if avg_ns else "- rocprof: n/a",
              f"- rocprof per-dispatch median {med_ns / 1e3:.3f} us, 10th percentile "
              f"{p10_ns / 1e3:.3f} us over {len(durs)} dispatches (start-to-end timestamps, "
              f"which include each dispatch's completion signal under tracing)" if durs else "",
              f"- algorithmic bytes per call: {bench['bytes']['algorithmic']}",
              f"- effective bandwidth: {bench['value']} GB/s ({bench['pct_hbm_peak']} % of 8 TB/s)", "",
              "## HBM traffic (rocprofv3 --pmc, one counter per run, KiB per dispatch)", "",
              f"- forward FETCH_SIZE {fwd_fetch}, WRITE_SIZE {fwd_write}",
              f"- plain copy of {copy_kib} KiB: FETCH_SIZE {copy_fetch}, WRITE_SIZE {copy_write}",
              f"- calibration factors: fetch {f_scale}, write {w_scale}",
              f"- forward HBM bytes per call (calibrated): {traffic}",
              f"- kernel source sha256[:16]: {bench['secondary']['kernel_sha256_16']}", ""]
    extra = {}
    for d in args.pmc_dirs:
        for r in _read_csv(d, "counter_collection.csv"):
            if "bev_pool_fwd" in r["Kernel_Name"]:
                extra.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    if extra:
        lines += ["## Further counters (rocprofv3 --pmc, mean per dispatch of the forward kernel)", ""]
        for k in sorted(extra):
            lines.append(f"- {k}: {sum(extra[k]) / len(extra[k]):.4g}")
        if "TCC_HIT_sum" in extra and "TCC_MISS_sum" in extra:
            hit, miss = sum(extra["TCC_HIT_sum"]), sum(extra["TCC_MISS_sum"])
            lines.append(f"- L2 (TCC) hit rate: {100 * hit / max(hit + miss, 1):.1f} %")
        lines.append("")
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    out_md = os.path.join(ROOT, "profiles", f"{name}_{workload}.md")
    with open(out_md, "w") as f:
        f.write("\n".join(lines))
    rec = {}
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    rec[workload] = {"kernel_sha256_16": bench["secondary"]["kernel_sha256_16"],
                     "hbm_bytes_per_launch": traffic, "fetch_kib": fwd_fetch, "write_kib": fwd_write,
                     "copy_calibration": {"kib": copy_kib, "fetch_kib": copy_fetch,
                                          "write_kib": copy_write},
                     "rocprof_avg_ns": avg_ns, "rocprof_median_ns": med_ns}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1, sort_keys=True)
    print(f"wrote {out_md} and {TRAFFIC_FILE}")


def cpu_baseline(wl, b_alg, seconds):
    """The oracle's scatter-reduce timed on the host, on a map it builds
    itself from the same seeded geometry."""
    import oracle
    oracle.build(force=False)
    s = wl.spec
    tm = time.perf_counter()
    ref_map = oracle.build_map(wl.point_cell, s.n_img, s.D, s.H, s.W, s.n_cells)
    map_ms = (time.perf_counter() - tm) * 1e3
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.forward(wl.depth, wl.feat, s.feat_dtype, wl.feat_scale, s.C, ref_map, s.n_cells)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    per = el / reps
    return {"value": round(b_alg / per / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{reps} full passes of the oracle's fp64 scatter-reduce over the "
                      f"{s.name} workload (N={ref_map['n_points']}), {el:.1f} s, single thread",
            "us_per_call": round(per * 1e6, 1),
            "map_build_ms": round(map_ms, 1),
            "cpu": _cpu_model()}


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def copy_calibration(mib, dev):
    """A plain streaming copy of known size (read mib MiB, write mib MiB) for
    calibrating the FETCH_SIZE / WRITE_SIZE counters of the same run."""
    import torch
    if not mib:
        return
    src = torch.empty(mib << 20, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(10):
        torch.bitwise_not(src, out=dst)
    torch.cuda.synchronize()


def bench_bags(args):
    """Weighted embedding bags through bevpool_segment_reduce (the same owner
    kernel); algorithmic bytes N*(C*e_table + e_weight + 4) + 4*(bags + 1) +
    bags*C*4."""
    import numpy as np
    import torch

    import depth_weighted_scatter_amd as dws
    import workloads

    dev = torch.device("cuda:0")
    b = workloads.make_bags(args.bags, args.seed)
    s = b.spec
    N = int(b.indices.size)
    w = torch.from_numpy(b.weights).to(dev) if b.weights is not None else None
    table = torch.from_numpy(b.table).to(dev)
    idx = torch.from_numpy(b.indices).to(dev)
    off = torch.from_numpy(b.offsets).to(dev)
    out = torch.empty((s.n_bags, s.C), dtype=torch.float32, device=dev)
    e_w = 0 if w is None else w.element_size()
    b_alg = N * (s.C * ELEM_BYTES[s.table_dtype] + e_w + 4) + 4 * (s.n_bags + 1) + s.n_bags * s.C * 4
    lib = dws._load()
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        dws.bevpool_segment_reduce(w, table, idx, off, b.table_scale, out)
    K = args.steps
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if args.eager:
        chunk = None
        a = dws.segment_reduce_args(w, table, idx, off, out, b.table_scale, stream)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(K):
            if lib.bevpool_segment_reduce(*a) != 0:
                raise RuntimeError("bevpool_segment_reduce failed")
        e1.record(stream)
        torch.cuda.synchronize()
    else:
        chunk = max(1, min(args.graph_chunk, K))
        while K % chunk:
            chunk -= 1
        cap = torch.cuda.Stream()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=cap):
            a = dws.segment_reduce_args(w, table, idx, off, out, b.table_scale, cap)
            for _ in range(chunk):
                if lib.bevpool_segment_reduce(*a) != 0:
                    raise RuntimeError("bevpool_segment_reduce failed")
        graph.replay()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(K // chunk):
            graph.replay()
        e1.record(stream)
        torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / K
    gbs = b_alg / (ms * 1e-3) / 1e9
    copy_calibration(args.copy_calib_mib, dev)
    print(json.dumps({
        "metric": "bevpool_segment_reduce µs/call + effective GB/s (% HBM peak), weighted embedding bags",
        "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": round(ms, 6), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32",
        "data": "synthetic (geometric bag lengths, skewed rows, N(0,1) table)",
        "config": {"workload": s.name, "bags": s.n_bags, "points": N, "table_rows": s.n_rows,
                   "C": s.C, "table_dtype": s.table_dtype, "weighted": w is not None,
                   "timing": "eager" if chunk is None else f"hip graph replay, {chunk} calls per graph"},
        "us_per_call": round(ms * 1e3, 3), "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic_for(s.name)},
        "bytes": {"algorithmic": b_alg},
        "secondary": {"copy_calib_mib": args.copy_calib_mib, "kernel_sha256_16": kernel_hash()}}),
        flush=True)


def main():
    args = parse()
    if args.summarize:
        summarize(args)
        return
    if args.bags is not None:
        if args.gpus != 1:
            print("bench.py runs on one GPU only", file=sys.stderr)
            sys.exit(2)
        bench_bags(args)
        return
    if args.out_dtype != "f32" and args.kernel != "owned":
        print("--out-dtype applies to the owned kernel only", file=sys.stderr)
        sys.exit(2)
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the pooled forward has no cross-GPU step "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import depth_weighted_scatter_amd as dws
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    wl = workloads.make_workload(args.workload, args.seed)
    s = wl.spec

    # inputs resident in HBM; map built once (timed separately)
    point_cell = torch.from_numpy(wl.point_cell).to(dev)
    depth = torch.from_numpy(wl.depth).to(dev)
    feat = torch.from_numpy(wl.feat).to(dev)
    out_torch = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[args.out_dtype]
    out = torch.empty((s.n_cells, s.C), dtype=out_torch, device=dev)
    m = dws.bevpool_build_map(point_cell, s.n_img, s.D, s.H, s.W, s.n_cells)   # warm
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    m = dws.bevpool_build_map(point_cell, s.n_img, s.D, s.H, s.W, s.n_cells)
    map_ms = (time.perf_counter() - t0) * 1e3
    N, I = m.n_points, m.n_intervals
    b_alg, b_min = algorithmic_bytes(s, N, I, out.element_size())

    lib = dws._load()
    stream = torch.cuda.current_stream()
    narrow = args.out_dtype != "f32"
    make_args = dws.forward_ex_args if narrow else dws.forward_args
    fargs = make_args(depth, feat, m, s.n_cells, out, wl.feat_scale, stream)

    order = {"v2": dws.ORDER_TILE_OUTER, "v2do": dws.ORDER_DEPTH_OUTER}.get(args.kernel)

    def call(a):
        if narrow:
            return lib.bevpool_forward_ex(*a)
        if order is None:
            return lib.bevpool_forward(*a)
        return lib.bevpool_forward_baseline(order, *a)

    def launch():
        rc = call(fargs)
        if rc != 0:
            raise dws.BevPoolError("bevpool_forward", rc)

    for _ in range(args.warmup):
        launch()
    torch.cuda.synchronize()

    K = args.steps
    chunk = max(1, min(args.graph_chunk, K))
    while K % chunk:
        chunk -= 1
    graph = None
    if not args.eager:
        cap_stream = torch.cuda.Stream()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=cap_stream):
            gargs = make_args(depth, feat, m, s.n_cells, out, wl.feat_scale, cap_stream)
            for _ in range(chunk):
                rc = call(gargs)
                if rc != 0:
                    raise dws.BevPoolError("bevpool_forward", rc)
        for _ in range(2):
            graph.replay()
        torch.cuda.synchronize()

    def timed(n_steps):
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        ev0.record(stream)
        if graph is not None:
            for _ in range(n_steps // chunk):
                graph.replay()
        else:
            for _ in range(n_steps):
                launch()
        ev1.record(stream)
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1)   # ms

    # torch.cuda.graph replays on the current stream, where the events sit
    t_wall0 = time.perf_counter()
    ms_total = timed(K)
    wall_s = time.perf_counter() - t_wall0
    ms_per_step = ms_total / K
    us = ms_per_step * 1e3
    gbs = b_alg / (ms_per_step * 1e-3) / 1e9

    # secondary: median of 100 trials of 20 calls, and eager back-to-back calls
    trials = []
    if graph is not None and chunk >= 1:
        per_trial = chunk * max(1, 20 // chunk) if chunk <= 20 else chunk
        for _ in range(100):
            trials.append(timed(per_trial) / per_trial * 1e3)
    eager_us = None
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(200):
        launch()
    ev1.record(stream)
    torch.cuda.synchronize()
    eager_us = ev0.elapsed_time(ev1) / 200 * 1e3

    # single-call latency (warm) and cold-cache latency: before each cold call a
    # 512 MiB buffer is overwritten, which evicts the 256 MB Infinity Cache and
    # the L2s, so inputs, map and output come from HBM
    def one_call_us(flush=None):
        if flush is not None:
            flush.fill_(0)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        launch()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3

    single = [one_call_us() for _ in range(100)]
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    cold = [one_call_us(flush) for _ in range(30)]
    del flush

    copy_calibration(args.copy_calib_mib, dev)

    workload_key = s.name if not narrow else f"{s.name}_out_{args.out_dtype}"
    traffic = traffic_for(workload_key)
    result = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",     # accumulation type; storage types are in config
        "data": "synthetic (seeded camera-frustum geometry; N(0,1) features, softmax depth)",
        "config": {"workload": workload_key, "cameras": s.n_cam, "frames": s.frames, "D": s.D,
                   "H": s.H, "W": s.W, "C": s.C, "bev_grid": [s.frames, s.G, s.G],
                   "scatter_points": N, "intervals": I, "feat_dtype": s.feat_dtype,
                   "depth_dtype": s.depth_dtype, "out_dtype": args.out_dtype,
                   "kernel": args.kernel,
                   "timing": "eager" if graph is None else
                   f"hip graph replay, {chunk} calls per graph"},
        "us_per_call": round(us, 3),
        "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic},
        "bytes": {"algorithmic": b_alg, "compulsory": b_min,
                  "compulsory_GBps": round(b_min / (ms_per_step * 1e-3) / 1e9, 2)},
        "secondary": {"median_us_100x20": round(float(np.median(trials)), 3) if trials else None,
                      "p10_us": round(float(np.percentile(trials, 10)), 3) if trials else None,
                      "p90_us": round(float(np.percentile(trials, 90)), 3) if trials else None,
                      "eager_back_to_back_us": round(eager_us, 3),
                      "single_call_us_median": round(float(np.median(single)), 3),
                      "cold_call_us_median": round(float(np.median(cold)), 3),
                      "cold_GBps": round(b_alg / (float(np.median(cold)) * 1e-6) / 1e9, 1),
                      "map_build_ms": round(map_ms, 3),
                      "timed_region_wall_s": round(wall_s, 3),
                      "copy_calib_mib": args.copy_calib_mib,
                      "kernel_sha256_16": kernel_hash()},
    }
    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(wl, b_alg, args.cpu_seconds)
    if args.details:
        with open(args.details, "w") as f:
            json.dump(result, f, indent=1)
    print(json.dumps(result), flush=True)
    if not math.isfinite(gbs):
        sys.exit(1)


if __name__ == "__main__":
    main()
