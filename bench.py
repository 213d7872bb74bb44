"""Benchmark of one MoE layer step on one MI355X.

A step is one moe_layer_forward over one batch of synthetic tokens: router GEMM,
top-k, routing tables, gate/up grouped GEMM with SwiGLU, down grouped GEMM,
shared expert and combine. Inputs are resident in HBM before the timed region.

Every timed layer reads its weights in the prepacked layout (moe_prepack_q4,
run once before timing, as a model load would); canonical_layout repeats the
T=4096 layer on the canonical layout for comparison (--layout canonical times
everything on it).

Prints one JSON line: value = tokens/s of the T=4096 layer, roofline = the
gate/up grouped GEMM (the dominant kernel) against the bf16 dense MFMA peak,
cpu_baseline = the fp64 oracle on the host cores, decode = the T=1 and T=8
layer as HBM bytes per second (weights rotated over 8 device-resident layer
sets so that the 256 MB last-level cache cannot hold the working set),
quantize = the 4-bit quantiser over one 256 x 512 x 2048 bf16 expert stack as
HBM bytes per second, prefill = the same layer at T=512, at T=4096 with a
Zipf(1.2) logit skew, and at T=32768, as tokens/s and % of the MFMA peak.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer prefill tokens/s @T=4096 (+% MFMA peak); decode-step HBM GB/s"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E


RAMP_SECONDS = 0.3


def ramp(torch, fn, seconds=None):
    """Call fn (a layer call or a graph replay) until `seconds` of wall time
    have passed, synchronising every few calls. The GPU raises its clocks under
    sustained load and takes tens of milliseconds to settle (the first ~50
    T=4096 layer calls ran 5-15% slower); the timed regions measure the
    sustained state. Returns the number of calls."""
    seconds = RAMP_SECONDS if seconds is None else seconds
    n = 0
    t0 = time.perf_counter()
    while True:
        for _ in range(4):
            fn()
            n += 1
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= seconds:
            return n


def layer_flops(T, H, I, E, k):
    return T * (2 * H * E + (k + 1) * 2 * H * 3 * I)


def gateup_flops(T, H, I, k):
    # real (token, expert) rows of the gate/up GEMM: T*k routed + T shared
    return (T * k + T) * 2 * H * (2 * I)


def q4_bytes(N, K):
    return N * K // 2 + 4 * N * (K // 64)


PER_EXPERT_BYTES = 3 * q4_bytes(512, 2048)    # gate, up, down of one expert at H=2048, I=512


def random_weights(ops, torch, dev, E, H, I, seed):
    """A layer of random weights drawn on the device (same distributions as the
    synthetic host generator: uniform codes, s = |N(0,1)|*0.02, b = -8s)."""
    g = torch.Generator(device=dev)
    g.manual_seed(seed)

    def stack(n, N, K):
        q = torch.randint(-2**31, 2**31 - 1, (n, N, K // 8), dtype=torch.int32, device=dev, generator=g)
        sc = (torch.randn(n, N, K // 64, device=dev, generator=g).abs() * 0.02).to(torch.bfloat16)
        b = (sc.float() * -8.0).to(torch.bfloat16)
        return ops.Q4Stack(q, sc, b)

    rw = (torch.randn(E, H, device=dev, generator=g) / math.sqrt(H)).to(torch.bfloat16)
    return ops.MoEWeights(router_w=rw, gate=stack(E, I, H), up=stack(E, I, H), down=stack(E, H, I),
                          sh_gate=stack(1, I, H), sh_up=stack(1, I, H), sh_down=stack(1, H, I))


def decode_measure(lib, _lib, ops, torch, dev, w0, T, k, n_sets=8, calls=16, reps=25, prepack=False,
                   persistent=False):
    """Layer calls at T tokens, captured as one HIP graph of `calls` calls that
    cycle over n_sets weight sets and `calls` fresh inputs, replayed `reps`
    times; bytes per call = the distinct experts the call routes to, plus the
    shared expert, the router matrix, x and y. prepack: every set (w0
    included) is prepacked before timing. persistent: the calls ask for the
    one-launch persistent decode kernel (moe_layer_forward_ex option)."""
    import ctypes
    E, H, I = w0.E, w0.H, w0.I
    sets = [w0] + [random_weights(ops, torch, dev, E, H, I, 1000 + i) for i in range(n_sets - 1)]
    if prepack:
        sets = [ws.prepacked() for ws in sets]
    structs = [[s.c_struct() for s in (w.gate, w.up, w.down, w.sh_gate, w.sh_up, w.sh_down)] for w in sets]
    gx = torch.Generator(device=dev)
    gx.manual_seed(77)
    xs = [torch.randn(T, H, device=dev, generator=gx).to(torch.bfloat16) for _ in range(calls)]
    ys = [torch.empty(T, H, dtype=torch.bfloat16, device=dev) for _ in range(calls)]
    ids = [torch.empty(T, k, dtype=torch.int32, device=dev) for _ in range(calls)]
    dims = _lib.MoeDims(T, H, I, E, k, 0)
    ws = torch.zeros(int(lib.moe_workspace_bytes(ctypes.byref(dims))), dtype=torch.uint8, device=dev)

    opts = _lib.MoeLayerOptions()
    opts.persistent_decode = 1 if persistent else 0

    def call(i):
        w = sets[i % n_sets]
        st = lib.moe_layer_forward_ex(
            ctypes.c_void_p(xs[i].data_ptr()), ctypes.c_void_p(w.router_w.data_ptr()), None,
            *[ctypes.byref(s) for s in structs[i % n_sets]], ctypes.byref(dims), ctypes.c_void_p(ys[i].data_ptr()),
            None, ctypes.c_void_p(ids[i].data_ptr()), None, ctypes.c_void_p(ws.data_ptr()), ws.numel(),
            ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream), ctypes.byref(opts))
        _lib.check(st, "moe_layer_forward_ex")

    for i in range(calls):
        call(i)
    torch.cuda.synchronize()
    eager = [y.clone() for y in ys]
    t0 = time.perf_counter()
    for i in range(calls):
        call(i)
    torch.cuda.synchronize()
    eager_us = (time.perf_counter() - t0) * 1e6 / calls
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(calls):
            call(i)
    graph.replay()
    torch.cuda.synchronize()
    ramp(torch, graph.replay)
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (reps * calls)
    same = all(torch.equal(a, b) for a, b in zip(eager, ys))
    distinct = [len(set(t.flatten().tolist())) for t in ids]
    bytes_per_call = [(d + 1) * PER_EXPERT_BYTES + E * H * 2 + 2 * T * H * 2 for d in distinct]
    avg_bytes = float(np.mean(bytes_per_call))
    gbs = avg_bytes / (us * 1e-6) / 1e9
    return {"T": T, "us_per_layer": us, "GB_per_s": gbs, "frac_hbm": gbs / PEAK_HBM_GBS,
            "bytes_per_layer": avg_bytes, "distinct_experts_avg": float(np.mean(distinct)),
            "eager_us_per_layer": eager_us, "graph_replay_matches_eager": bool(same),
            "method": f"HIP graph of {calls} layer calls over {n_sets} weight sets and {calls} inputs, "
                      f"{reps} replays timed with events"}


def prefill_measure(lib, _lib, ops, torch, dev, w, T, k, zipf=None, steps=10, warmup=3, weight_bytes=None):
    """Layer calls at T tokens on the same layer weights (x drawn on the device,
    N(0,1) in bf16; optional Zipf logit bias -zipf*ln(e+1)): `steps` calls
    launched back to back and timed with events (ms_per_layer), and the same
    calls captured in one HIP graph and replayed (graph_ms_per_layer)."""
    import ctypes
    E, H, I = w.E, w.H, w.I
    g = torch.Generator(device=dev)
    g.manual_seed(11 + T)
    x = torch.randn(T, H, device=dev, generator=g).to(torch.bfloat16)
    y = torch.empty(T, H, dtype=torch.bfloat16, device=dev)
    bias = None
    if zipf is not None:
        bias = (-float(zipf) * torch.log(torch.arange(1, E + 1, dtype=torch.float64))).to(torch.float32).to(dev)
    ids = torch.empty(T, k, dtype=torch.int32, device=dev)
    structs = [s.c_struct() for s in (w.gate, w.up, w.down, w.sh_gate, w.sh_up, w.sh_down)]
    dims = _lib.MoeDims(T, H, I, E, k, 0)
    ws = torch.zeros(int(lib.moe_workspace_bytes(ctypes.byref(dims))), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def call():
        st = lib.moe_layer_forward(
            ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(w.router_w.data_ptr()),
            ctypes.c_void_p(bias.data_ptr()) if bias is not None else None,
            *[ctypes.byref(s) for s in structs], ctypes.byref(dims), ctypes.c_void_p(y.data_ptr()),
            None, ctypes.c_void_p(ids.data_ptr()), None, ctypes.c_void_p(ws.data_ptr()), ws.numel(),
            ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream))
        _lib.check(st, "moe_layer_forward")

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    ramp(torch, call)
    y_eager = y.clone()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(steps):
            call()
    graph.replay()
    torch.cuda.synchronize()
    same = bool(torch.equal(y, y_eager))
    ramp(torch, graph.replay)   # the GPU idled during the capture
    e0.record(stream)
    graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    graph_ms = e0.elapsed_time(e1) / steps
    del graph
    counts = torch.bincount(ids.flatten().long(), minlength=E).cpu().numpy()
    flops = layer_flops(T, H, I, E, k)
    out = {"T": T, "ms_per_layer": ms, "tokens_per_s": T / (ms * 1e-3),
           "pct_mfma_peak": 100.0 * flops / (ms * 1e-3) / (PEAK_BF16_TFLOPS * 1e12),
           "logit_bias": f"zipf{zipf}" if zipf is not None else None,
           "experts_hit": int((counts > 0).sum()), "max_rows_per_expert": int(counts.max()),
           "graph_ms_per_layer": graph_ms, "graph_replay_matches_eager": same,
           "method": f"{steps} back-to-back layer calls timed with events at sustained clocks; graph: the same "
                     f"calls captured in one HIP graph and replayed"}
    if weight_bytes:
        # weights of the experts this call routed to (+ shared, + router), as HBM bytes per second
        hit = int((counts > 0).sum())
        nbytes = (hit + 1) * PER_EXPERT_BYTES + E * H * 2 + 2 * T * H * 2
        out["weight_and_io_bytes"] = nbytes
        out["GB_per_s"] = nbytes / (ms * 1e-3) / 1e9
        out["frac_hbm"] = out["GB_per_s"] / PEAK_HBM_GBS
    del x, y, ws, ids
    return out


def quantize_measure(ops, torch, dev, n=256, N=512, K=2048, reps=10):
    """The quantiser over one whole expert weight stack (n experts of N x K bf16,
    the gate stack of the layer) timed with events on the launch stream; bytes =
    the bf16 weights read plus codes, scales and offsets written."""
    g = torch.Generator(device=dev)
    g.manual_seed(5)
    w = (torch.randn(n, N, K, device=dev, generator=g) * 0.02).to(torch.bfloat16)
    out = ops.quantize_q4(w)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        ops.quantize_q4(w, out)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    nbytes = n * N * K * 2 + q4_bytes(n * N, K)
    gbs = nbytes / (us * 1e-6) / 1e9
    del w, out
    return {"kernel": "quantize_q4_kernel", "shape": [n, N, K], "us": us, "bytes": nbytes,
            "GB_per_s": gbs, "frac_hbm": gbs / PEAK_HBM_GBS, "bound": "hbm",
            "method": f"{reps} back-to-back calls timed with events"}


TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "gemm_q4_swiglu_prefill4096_traffic.txt")
KERNEL_SOURCES = ("int4_expert_routing_amd/csrc/gemm_q4.hip", "int4_expert_routing_amd/csrc/gemm_tiles.h",
                  "int4_expert_routing_amd/csrc/gemm_args.h", "int4_expert_routing_amd/csrc/moe_common.h")
GEMM_KERNEL_NAME = "gemm_q4_kernel<2, 2>"


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_traffic():
    """HBM bytes per gate/up launch from the committed counter summary, if it
    was taken on the current kernel source (else None)."""
    try:
        kv = dict(line.split("=", 1) for line in open(TRAFFIC_SUMMARY).read().splitlines()
                  if "=" in line and not line.startswith(" "))
    except OSError:
        return None
    if kv.get("source_hash", "").strip() != kernel_source_hash():
        return None
    return float(kv["traffic_bytes_per_launch"])


def counter_values(run_dir, counter, by_grid=False):
    """{dispatch kernel name (and grid size): [value per dispatch]} from a rocprofv3 --pmc csv run."""
    import csv
    import glob
    out = {}
    for f in glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] == counter:
                key = (r["Kernel_Name"], int(r["Grid_Size"])) if by_grid else r["Kernel_Name"]
                out.setdefault(key, []).append(float(r["Counter_Value"]))
    return out


def write_counter_summary(out_path, title, fetch_dir, write_dir, copy_mib, cmd_fetch, cmd_write):
    """HBM bytes per dispatch of every library kernel in two rocprofv3 --pmc runs
    (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch), grouped by kernel and grid
    size, each counter scaled by what it reads for the calibration copy kernel
    of copy_mib MiB (read and written once) in the same run."""
    fv, wv = counter_values(fetch_dir, "FETCH_SIZE", True), counter_values(write_dir, "WRITE_SIZE", True)
    c_f = [v for (kname, _), vs in fv.items() if "copyBuffer" in kname for v in vs]
    c_w = [v for (kname, _), vs in wv.items() if "copyBuffer" in kname for v in vs]
    if not (c_f and c_w):
        raise SystemExit("calibration copy kernel missing from the counter runs")
    true_bytes = copy_mib * 2**20
    f_scale = true_bytes / (max(c_f) * 1024.0)
    w_scale = true_bytes / (max(c_w) * 1024.0)
    lines = [title, f"  FETCH_SIZE pass: {cmd_fetch}", f"  WRITE_SIZE pass: {cmd_write}",
             f"  calibration copy kernel: {copy_mib} MiB read + written once; counter reads FETCH {max(c_f):.0f} KiB, "
             f"WRITE {max(c_w):.0f} KiB -> scale fetch {f_scale:.4f}, write {w_scale:.4f}",
             f"  {'kernel':58s} {'grid':>9s} {'n':>4s} {'fetch MB':>10s} {'write MB':>10s}  (median per dispatch)"]
    for key in sorted(fv, key=lambda kk: (kk[0], kk[1])):
        kname, grid = key
        if "moe::" not in kname or key not in wv:
            continue
        fb = float(np.median(fv[key])) * 1024.0 * f_scale
        wb = float(np.median(wv[key])) * 1024.0 * w_scale
        short = kname.replace("void ", "").split("(")[0]
        lines.append(f"  {short[:58]:58s} {grid:9d} {len(fv[key]):4d} {fb / 1e6:10.3f} {wb / 1e6:10.3f}")
    lines.append(f"source_hash={kernel_source_hash()}")
    with open(out_path, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def write_traffic_summary(fetch_dir, write_dir, copy_mib, cmd_fetch, cmd_write):
    """Gate/up HBM traffic per launch from FETCH_SIZE and WRITE_SIZE (KiB per
    dispatch), each scaled by what the counter reads for the calibration copy
    kernel of copy_mib MiB (read and written once)."""
    fv, wv = counter_values(fetch_dir, "FETCH_SIZE"), counter_values(write_dir, "WRITE_SIZE")
    pick = lambda d, key: [v for k, vs in d.items() if key in k for v in vs]
    g_f, g_w = pick(fv, GEMM_KERNEL_NAME), pick(wv, GEMM_KERNEL_NAME)
    c_f, c_w = pick(fv, "copyBuffer"), pick(wv, "copyBuffer")
    if not (g_f and g_w and c_f and c_w):
        raise SystemExit(f"counters missing: gemm {len(g_f)}/{len(g_w)}, copy {len(c_f)}/{len(c_w)}")
    true_bytes = copy_mib * 2**20
    f_scale = true_bytes / (max(c_f) * 1024.0)
    w_scale = true_bytes / (max(c_w) * 1024.0)
    fetch = float(np.median(g_f)) * 1024.0 * f_scale
    write = float(np.median(g_w)) * 1024.0 * w_scale
    lines = [
        "gate/up grouped GEMM (gemm_q4_kernel<SwiGLU>), T=4096 layer: HBM traffic per launch",
        f"  FETCH_SIZE pass: {cmd_fetch}",
        f"  WRITE_SIZE pass: {cmd_write}",
        f"  calibration copy kernel: {copy_mib} MiB read + written once; counter reads "
        f"FETCH {max(c_f):.0f} KiB, WRITE {max(c_w):.0f} KiB -> scale fetch {f_scale:.4f}, write {w_scale:.4f}",
        f"  gate/up dispatches: {len(g_f)}; median FETCH {np.median(g_f):.0f} KiB, WRITE {np.median(g_w):.0f} KiB",
        f"fetch_bytes_per_launch={fetch:.0f}",
        f"write_bytes_per_launch={write:.0f}",
        f"traffic_bytes_per_launch={fetch + write:.0f}",
        f"source_hash={kernel_source_hash()}",
    ]
    with open(os.environ.get("TRAFFIC_SUMMARY_OUT", TRAFFIC_SUMMARY), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--ramp-seconds", type=float, default=RAMP_SECONDS,
                   help="untimed calls before each timed region, in seconds of wall time (sustained clocks)")
    p.add_argument("--config", default="prefill4096")
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-decode", action="store_true")
    p.add_argument("--no-quantize", action="store_true")
    p.add_argument("--no-prefill-sweep", action="store_true")
    p.add_argument("--no-side-stream", action="store_true",
                   help="skip the timing of the calls with the shared expert on a second stream")
    p.add_argument("--layout", choices=("prepacked", "canonical"), default="prepacked",
                   help="weight layout of every timed layer (prepacked once, before timing)")
    p.add_argument("--calib-copy-mib", type=int, default=0,
                   help="after the timed steps, launch one device copy of this many MiB (counter calibration)")
    p.add_argument("--write-traffic-summary", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "CMD_FETCH", "CMD_WRITE"),
                   help="build the gate/up traffic summary from two rocprofv3 --pmc runs and exit")
    p.add_argument("--write-counter-summary", nargs=6,
                   metavar=("OUT", "TITLE", "FETCH_DIR", "WRITE_DIR", "CMD_FETCH", "CMD_WRITE"),
                   help="per-kernel HBM bytes per dispatch from two rocprofv3 --pmc runs, and exit")
    return p.parse_args()


def cpu_baseline(inp, small):
    """Time the fp64 oracle as it stands: the median of 3 full layer passes over
    the timed workload with every BLAS thread, and one single-thread pass over
    the T=512 workload."""
    import oracle.moe_oracle as om
    from threadpoolctl import threadpool_info, threadpool_limits
    blas = max([int(i.get("num_threads", 1)) for i in threadpool_info()] or [1])
    runs = []
    for _ in range(3):
        t0 = time.perf_counter()
        om.moe_layer(inp)
        runs.append(time.perf_counter() - t0)
    dt = float(np.median(runs))
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        om.moe_layer(small)
        dt1 = time.perf_counter() - t0
    return {"value": inp.T / dt, "unit": "tokens/s", "cores": blas, "host_cpu_count": os.cpu_count(),
            "blas_threads": blas, "kind": "oracle",
            "sample": f"full layer passes over the T={inp.T} workload (all of it), median of 3: "
                      f"{', '.join(f'{r:.2f}' for r in runs)} s",
            "seconds": dt,
            "single_thread_T512": {"value": small.T / dt1, "unit": "tokens/s", "cores": 1, "seconds": dt1,
                                   "sample": f"one full layer pass, T={small.T}, BLAS limited to 1 thread"}}


def main():
    args = parse()
    global RAMP_SECONDS
    RAMP_SECONDS = args.ramp_seconds
    if args.write_traffic_summary:
        fd, wd, cf, cw = args.write_traffic_summary
        write_traffic_summary(fd, wd, 512, cf, cw)
        return
    if args.write_counter_summary:
        op_, title, fd, wd, cf, cw = args.write_counter_summary
        write_counter_summary(op_, title, fd, wd, 512, cf, cw)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported: this library runs on a "
              "single GPU (with the weights replicated, the layer shards over tokens with no exchange, "
              "so N GPUs would each run this benchmark on their own tokens)", file=sys.stderr)
        sys.exit(2)
    import ctypes

    import torch

    from int4_expert_routing_amd import _lib, ops
    from synth import CONFIGS, make_config

    lib = _lib.load()
    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    dev = torch.device("cuda:0")
    cfg = CONFIGS[args.config]
    inp = make_config(args.config, seed=args.seed)
    T, H, I, E, k = inp.T, inp.H, inp.I, inp.E, inp.k
    w_canon = ops.MoEWeights.from_host(inp, dev)
    packed = args.layout == "prepacked"
    w = w_canon.prepacked() if packed else w_canon
    x = ops.bf16_from_bits(inp.x, dev)
    layer = ops.MoELayer(w, k, T)
    y = torch.empty(T, H, dtype=torch.bfloat16, device=dev)
    structs = [s.c_struct() for s in (w.gate, w.up, w.down, w.sh_gate, w.sh_up, w.sh_down)]
    dims = _lib.MoeDims(T, H, I, E, k, 0)
    nev = _lib.MOE_LAYER_STAGE_EVENTS
    stream = torch.cuda.current_stream(dev)

    def step(events=None):
        evp = None
        n = 0
        if events is not None:
            evp = (ctypes.c_void_p * nev)(*[e.cuda_event for e in events])
            n = nev
        st = lib.moe_layer_forward_timed(
            ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(w.router_w.data_ptr()),
            ctypes.c_void_p(w.logit_bias.data_ptr()) if w.logit_bias is not None else None,
            *[ctypes.byref(s) for s in structs], ctypes.byref(dims), ctypes.c_void_p(y.data_ptr()), None, None,
            None, ctypes.c_void_p(layer.workspace.data_ptr()), layer.workspace.numel(),
            ctypes.c_void_p(stream.cuda_stream), evp, n)
        _lib.check(st, "moe_layer_forward_timed")

    def plain_step():
        st = lib.moe_layer_forward(
            ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(w.router_w.data_ptr()),
            ctypes.c_void_p(w.logit_bias.data_ptr()) if w.logit_bias is not None else None,
            *[ctypes.byref(s) for s in structs], ctypes.byref(dims), ctypes.c_void_p(y.data_ptr()), None, None,
            None, ctypes.c_void_p(layer.workspace.data_ptr()), layer.workspace.numel(),
            ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream))
        _lib.check(st, "moe_layer_forward")

    for _ in range(args.warmup):
        plain_step()
    torch.cuda.synchronize()
    ramp_calls = ramp(torch, plain_step)
    # the timed region: K back-to-back layer calls between synchronizations
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        plain_step()
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    y_ref = y.clone()

    # the same calls with HIP events between the stages (stage times and the
    # gate/up launch's duration for the roofline)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(args.steps)]
    for e in evs:            # create the HIP events before use
        for ev in e:
            ev.record(stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(evs[s])
    torch.cuda.synchronize()
    events_ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    stage_ms = np.zeros(nev - 1)
    step_ms = []
    for e in evs:
        for i in range(nev - 1):
            stage_ms[i] += e[i].elapsed_time(e[i + 1])
        step_ms.append(e[0].elapsed_time(e[nev - 1]))
    stage_ms /= args.steps

    # and captured in one HIP graph (the whole layer as one submission, as the
    # pages' single command buffer), replayed once
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(args.steps):
            plain_step()
    graph.replay()   # untimed: the first replay uploads the graph
    torch.cuda.synchronize()
    graph_matches = bool(torch.equal(y, y_ref))
    ramp(torch, graph.replay)   # the GPU idled during the capture
    t0 = time.perf_counter()
    graph.replay()
    torch.cuda.synchronize()
    graph_ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    del graph

    # the same calls with the shared expert's GEMMs on a second stream (the
    # moe_layer_forward_ex side-stream option), reported beside the value
    side_ms_per_step, side_matches = None, None
    if not args.no_side_stream:
        side = ops.MoELayer(w, k, T, side_stream=True)
        y_side = torch.empty_like(y)
        side_call = lambda: side(x, y=y_side)
        side_call()
        torch.cuda.synchronize()
        ramp(torch, side_call)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            side_call()
        torch.cuda.synchronize()
        side_ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
        side_matches = bool(torch.equal(y_side, y_ref))
        del side
    gpu_ms = float(np.mean(step_ms))
    names = ["prep", "route", "gate_up_gemm", "down_gemm", "combine"]
    flops = layer_flops(T, H, I, E, k)
    gu_flops = gateup_flops(T, H, I, k)
    gu_ms = float(stage_ms[2])
    achieved_tflops = gu_flops / (gu_ms * 1e-3) / 1e12
    weight_bytes = E * 3 * q4_bytes(I, H) + 3 * q4_bytes(I, H) + E * H * 2
    out = {
        "metric": METRIC,
        "value": T / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{args.config}: MoE layer T={T} H={H} I={I} E={E} top-{k} + 1 shared expert, "
                               "int4 g64 affine weights (bf16 scale/bias), bf16 activations",
                   "T": T, "H": H, "I": I, "E": E, "k": k, "seed": args.seed,
                   "logit_bias": "zipf1.2" if cfg.get("zipf") else None,
                   "weight_layout": ("prepacked (moe_prepack_q4, once before timing)" if packed
                                     else "canonical")},
        "layer_pct_mfma_peak": 100.0 * flops / (ms_per_step * 1e-3) / (PEAK_BF16_TFLOPS * 1e12),
        "timing": (f"{args.steps} back-to-back layer calls, wall clock between synchronizations, after the "
                   f"{args.warmup} warm-up calls and {ramp_calls} more calls ({RAMP_SECONDS} s) that bring the GPU "
                   "to its sustained clocks; graph_ms_per_step: the same calls captured in one HIP graph and "
                   "replayed once; events_ms_per_step: with HIP events between the stages; "
                   "side_stream_ms_per_step: the same calls with the shared expert's GEMMs on a second stream"),
        "graph_ms_per_step": graph_ms_per_step,
        "side_stream_ms_per_step": side_ms_per_step,
        "side_stream_matches_one_stream": side_matches,
        "events_ms_per_step": events_ms_per_step,
        "graph_replay_matches_eager": graph_matches,
        "layer_gpu_ms_events": gpu_ms,
        "stage_ms": {n: float(v) for n, v in zip(names, stage_ms)},
        "roofline": {"kernel": "gemm_q4_kernel<SwiGLU> (gate/up grouped GEMM)", "bound": "mfma",
                     "achieved": achieved_tflops, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved_tflops / PEAK_BF16_TFLOPS, "traffic": read_traffic(),
                     "traffic_unit": "bytes per launch (HBM, FETCH_SIZE + WRITE_SIZE scaled by a copy kernel)",
                     "algorithmic_flops_per_launch": gu_flops},
        "weight_bytes": weight_bytes,
    }
    if args.calib_copy_mib:
        src = torch.empty(args.calib_copy_mib * 2**20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
    if packed and not args.no_prefill_sweep:
        # the same workload with the weights in the canonical layout
        c = prefill_measure(lib, _lib, ops, torch, dev, w_canon, T, k, zipf=cfg.get("zipf"))
        out["canonical_layout"] = {"ms_per_layer": c["ms_per_layer"], "tokens_per_s": c["tokens_per_s"],
                                   "method": c["method"]}
    if not args.no_decode:
        out["decode"] = {}
        for dname in ("decode1", "decode8"):
            dinp = make_config(dname, seed=args.seed)
            dw = ops.MoEWeights.from_host(dinp, dev)
            out["decode"][dname] = decode_measure(lib, _lib, ops, torch, dev, dw, dinp.T, dinp.k, prepack=packed)
            del dw
    if not args.no_prefill_sweep:
        out["prefill"] = {
            "prefill512": prefill_measure(lib, _lib, ops, torch, dev, w, 512, k, weight_bytes=True),
            "prefill4096_zipf": prefill_measure(lib, _lib, ops, torch, dev, w, 4096, k, zipf=1.2),
            "prefill32768": prefill_measure(lib, _lib, ops, torch, dev, w, 32768, k, steps=5, warmup=2),
        }
    if not args.no_quantize:
        out["quantize"] = quantize_measure(ops, torch, dev)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(inp, make_config("prefill512", seed=args.seed))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
