"""Benchmark of the W1.58A8 ternary linear layer hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--m M] [--split] [--row-scales] [--eager]
                    [--no-cpu-baseline]

A step is one pass of the whole per-call hot path over one batch of synthetic input:
for every resident weight matrix, quantize its fp32 activations per token to int8, run
the integer ternary product and apply the scale epilogue -- one bt_ternary_linear call
per matrix (a single fused kernel at decode sizes; bt_quant_act + bt_ternary_gemm_ws for
prefill, which splits K over several workgroups per tile where the tiles alone would
leave the GPU idle). ``--split`` times the same two launches called one by one
(bt_quant_act + bt_ternary_gemv / bt_ternary_gemm_ws) instead. ``--row-scales`` packs the
fused Q/K/V and gate/up matrices with one weight scale per block (bt_pack_weights_rows)
and runs the row-scale entry points. Weight packing is offline and outside the timed region. Inputs
are resident in HBM before timing starts; the step is replayed as one HIP graph.
Prints ONE JSON line.

Workloads (``--workload``):
  2b_decode   (default) 2B-class decode, M = 1: 30 layers x {QKV 3840x2560, O 2560x2560,
              gate+up 13824x2560, down 2560x6912}, all 120 packed matrices resident
              (521 MB, twice the 256 MB Infinity Cache) -> metric in GB/s.
  7b_decode   7B-class decode at --m (1, 4, 8): 32 layers of {12288x4096, 4096x4096,
              22016x4096, 4096x11008} resident (1.62 GB) -> GB/s.
  100b_decode 100B-class single-layer sweep at --m (1, 16): 3 independently seeded copies
              of {10240x8192, 8192x8192, 57344x8192, 8192x28672} (642 MB) -> GB/s.
  2b_prefill  2B-class prefill at --m (256, 2048): the 2B layer shapes, 30 layers -> TOPS.
  onebit_decode  1-bit activations (bit-floor page's GEMV shapes): 4096x4096 binary weights
              (bt_binary_gemv) and 4096x4096, 11008x4096 ternary weights
              (bt_ternary_gemv_a1), 30 copies resident, at --m (default 1) -> GB/s.

The dominant kernel's average duration comes from a second graph holding only the
product launches of one step (for the fused decode route that is the whole step),
timed with HIP events on the stream it runs on. HBM traffic per launch comes from a
committed rocprofv3 counter summary under profiles/ (see ``--summarize-pmc``) and is
reported only while the kernel sources still hash to the values recorded there.
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "ternary GEMV HBM GB/s (% of peak) at 2B decode shapes; prefill GEMM int8 TOPS"
HBM_PEAK_GBS = 8000.0    # MI355X HBM3E, 8 TB/s
INT8_PEAK_TOPS = 5000.0  # MI355X dense int8 MFMA, 5.0 POP/s
CSRC = os.path.join(ROOT, "bit_ternary_weight_absmean_amd", "csrc")
# Sources each dominant kernel is built from (their hash tags a traffic summary).
KERNEL_SOURCES = {
    "k_linear_decode": ["decode.hip", "wave.h", "bt_internal.h"],
    "k_gemv_direct": ["decode.hip", "wave.h", "bt_internal.h"],
    "k_gemv_staged": ["decode.hip", "wave.h", "bt_internal.h"],
    "k_gemv_dot4": ["gemv.hip", "bt_internal.h"],
    "k_gemv_lut": ["lut.hip", "bt_internal.h"],
    "k_gemm": ["gemm.hip", "bt_internal.h"],
}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="2b_decode", choices=["2b_decode", "7b_decode", "100b_decode", "2b_prefill",
                                                                   "onebit_decode"])
    p.add_argument("--m", type=int, default=None, help="tokens per call (default: 1 for decode, 2048 for prefill)")
    p.add_argument("--eager", action="store_true", help="launch kernels one by one instead of replaying graphs")
    p.add_argument("--split", action="store_true", help="time bt_quant_act + product as two launches per matrix")
    p.add_argument("--gemv-algo", choices=("auto", "mfma", "staged", "dot4", "lut"), default="auto",
                   help="at M <= 16 on the unfused route: the decode product kernel (bt_ternary_gemv_algo)")
    p.add_argument("--row-scales", action="store_true",
                   help="row-group weight scales: fused Q/K/V and gate/up matrices packed with one scale per "
                        "block (bt_pack_weights_rows), products through the row-scale entry points")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=10.0, help="target CPU time of the oracle baseline")
    p.add_argument("--calib-copy", action="store_true",
                   help="only run a plain 1 GiB device copy 10 times (HBM counter calibration)")
    p.add_argument("--summarize-pmc", nargs=5, metavar=("FETCH_DIR", "WRITE_DIR", "CAL_FETCH_DIR", "CAL_WRITE_DIR",
                                                        "OUT_JSON"),
                   help="write a traffic summary from rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE outputs of this "
                        "workload and of --calib-copy, for the workload's dominant kernel")
    p.add_argument("--summarize-mfma", nargs=2, metavar=("PMC_DIR", "OUT_JSON"),
                   help="write an MFMA-utilization summary for the prefill GEMM from a rocprofv3 --pmc "
                        "MfmaUtil SQ_INSTS_VALU_MFMA_MOPS_I8 run of this workload")
    p.add_argument("--command", default="", help="the rocprofv3 command line recorded with --summarize-pmc / -mfma")
    return p.parse_args()


# ----------------------------------------------------------------- workloads
def workload_spec(name, m):
    from bit_ternary_weight_absmean_amd import synth

    if name == "2b_decode":
        return dict(name=name, cfg=synth.CFG_2B_DECODE, shapes=synth.SHAPES_2B, layers=30, M=m or 1,
                    prefill=False, desc="2B-class decode GEMVs, 30 layers resident")
    if name == "7b_decode":
        return dict(name=name, cfg=synth.CFG_7B_DECODE, shapes=synth.SHAPES_7B, layers=32, M=m or 1,
                    prefill=False, desc="7B-class decode GEMVs, 32 layers resident")
    if name == "100b_decode":
        return dict(name=name, cfg=synth.CFG_100B_DECODE, shapes=synth.SHAPES_100B, layers=3, M=m or 1,
                    prefill=False, desc="100B-class single-layer decode sweep, 3 seeded copies resident")
    return dict(name=name, cfg=synth.CFG_2B_PREFILL, shapes=synth.SHAPES_2B, layers=30, M=m or 2048, prefill=True,
                desc="2B-class prefill GEMMs, 30 layers resident")


# Weight-scale bytes per call: one fp32 gamma, or N row scales with --row-scales.
ROW_SCALES = False


def scale_bytes(N):
    return 4 * N if ROW_SCALES else 4


def gemv_bytes(M, N, K):
    """Algorithmic HBM bytes of one product call on pre-quantized activations: 2-bit
    weights, int8 activations read, fp32 output written, weight scale(s) + s_x + sum q read."""
    return N * K // 4 + M * K + 4 * M * N + scale_bytes(N) + 8 * M


def linear_bytes(M, N, K):
    """Algorithmic HBM bytes of one fused call: 2-bit weights and fp32 activations read,
    fp32 output written, weight scale(s) read."""
    return N * K // 4 + 4 * M * K + 4 * M * N + scale_bytes(N)


def quant_bytes(M, K):
    """Algorithmic bytes of one activation quantization: fp32 read, int8 + s_x + sum q written."""
    return 4 * M * K + M * K + 8 * M


def source_hash(kernel):
    """SHA-256 of the kernel's sources with comments, indentation and blank lines taken out:
    counter figures stay valid across comment edits and are dropped on any code change."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, f), encoding="utf-8") as fh:
            text = re.sub(r"/\*.*?\*/", " ", fh.read(), flags=re.S)
        for line in text.splitlines():
            code = line.split("//", 1)[0].strip()
            if code:
                h.update(code.encode() + b"\n")
    return h.hexdigest()


def traffic_path(workload, kernel, M):
    return os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}_m{M}.json")


# ----------------------------------------------------------------- main leg
def run_gpu(args, spec):
    import torch

    import bit_ternary_weight_absmean_amd as bt
    from bit_ternary_weight_absmean_amd import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    M = spec["M"]
    shapes = spec["shapes"]
    cfg = spec["cfg"]

    # Resident packed weights (drawn on the device from seeded generators, packed, fp32 freed).
    packed = []
    ws = torch.empty(max(bt.pack_workspace_bytes(max(n for _, n, _ in shapes), 1), 8), dtype=torch.uint8,
                     device=dev)
    t0 = time.time()
    for layer in range(spec["layers"]):
        row = []
        for j, (name, N, K) in enumerate(shapes):
            W = synth.device_gaussian((N, K), synth.weight_seed(cfg, layer, j), dev, std=synth.WEIGHT_STD)
            if ROW_SCALES:
                row.append(bt.pack_weights_rows(W, synth.row_groups(cfg, name, N), workspace=ws))
            else:
                row.append(bt.pack_weights(W, workspace=ws))
            del W
        packed.append(row)
    torch.cuda.synchronize()
    setup_s = time.time() - t0
    resident = sum(p.data.numel() for row in packed for p in row)

    # Per-matrix-type activations, output buffers and (route permitting) workspaces.
    xs, qs, ys, wss, gws = [], [], [], [], []
    for j, (_, N, K) in enumerate(shapes):
        X = torch.from_numpy(synth.layer_activation(cfg, j, M, K)).to(dev)
        xs.append(X)
        qs.append(bt.quant_act(X))
        ys.append(torch.empty((M, N), dtype=torch.float32, device=dev))
        wb = bt.linear_workspace_bytes(M, N, K)
        wss.append(torch.empty(wb, dtype=torch.uint8, device=dev) if wb else None)
        # zero-filled split-K workspace for direct bt_ternary_gemm_ws calls (None: no split)
        gws.append(bt.gemm_workspace(M, N, K, dev) if M > bt.GEMV_MAX_M else None)
    torch.cuda.synchronize()

    fused = (not args.split) and all(bt.linear_workspace_bytes(M, N, K) == 0 for _, N, K in shapes)
    if fused:
        kernel = "k_linear_decode"
    elif spec["prefill"] or M > bt.GEMV_MAX_M:
        kernel = "k_gemm"
    else:
        names = {"mfma": "k_gemv_direct", "staged": "k_gemv_staged", "dot4": "k_gemv_dot4", "lut": "k_gemv_lut"}
        if args.gemv_algo == "auto":  # the library's pick per shape (BT_GEMV_AUTO), as bt_ternary_linear makes it
            picks = ["staged" if M * ((K + 255) // 256 * 256) <= 131072 else "mfma" for _, _, K in shapes]
            kernel = " + ".join(dict.fromkeys(names[c] for c in picks))
        else:
            kernel = names[args.gemv_algo]
    algo = {"auto": bt.GEMV_AUTO, "mfma": bt.GEMV_MFMA, "staged": bt.GEMV_STAGED, "dot4": bt.GEMV_DOT4,
            "lut": bt.GEMV_LUT}[args.gemv_algo]

    def product(pw, q, out_y, j):
        if kernel == "k_gemm":
            return bt.ternary_gemm(pw, q, out_y=out_y, workspace=gws[j])
        return bt.ternary_gemv(pw, q, out_y=out_y, algo=algo)

    def step():
        for row in packed:
            for j, pw in enumerate(row):
                if args.split:
                    bt.quant_act(xs[j], out=qs[j])
                    product(pw, qs[j], ys[j], j)
                else:
                    bt.linear(xs[j], pw, out_y=ys[j], workspace=wss[j])

    def products():
        """Only the dominant kernel's launches of one step (activations already quantized)."""
        for row in packed:
            for j, pw in enumerate(row):
                if fused:
                    bt.linear(xs[j], pw, out_y=ys[j])
                else:
                    product(pw, qs[j], ys[j], j)

    stream = torch.cuda.Stream(device=dev)

    def timed(fn, steps, warmup):
        run = fn
        if not args.eager:
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph, stream=stream):
                fn()
            stream.synchronize()
            run = graph.replay
        for _ in range(warmup):
            run()
        stream.synchronize()
        torch.cuda.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record(stream)
        for _ in range(steps):
            run()
        end.record(stream)
        end.synchronize()
        torch.cuda.synchronize()
        return start.elapsed_time(end) / steps

    with torch.cuda.stream(stream):
        for _ in range(2):  # eager warmup (library load, first touch)
            step()
        stream.synchronize()
        ms_step = timed(step, args.steps, args.warmup)
        ms_prod = ms_step if fused else timed(products, args.steps, args.warmup)

    step_bytes = step_ops = prod_bytes = 0
    for row in packed:
        for j, (_, N, K) in enumerate(shapes):
            # the fused kernel reads fp32 x once and never writes or re-reads int8 Xq
            if fused:
                step_bytes += linear_bytes(M, N, K)
                prod_bytes += linear_bytes(M, N, K)
            else:
                step_bytes += gemv_bytes(M, N, K) + quant_bytes(M, K)
                prod_bytes += gemv_bytes(M, N, K)
            step_ops += 2 * M * N * K
    n_prod = spec["layers"] * len(shapes)
    return dict(ms_step=ms_step, ms_prod=ms_prod, step_bytes=step_bytes, step_ops=step_ops,
                prod_bytes=prod_bytes, n_prod=n_prod, resident=resident, setup_s=setup_s,
                launch="eager" if args.eager else "hipGraph", fused=fused, kernel=kernel)


# ------------------------------------------------- 1-bit activations (W1A1, W1.58A1)
ONEBIT_COPIES = 30  # 30 x 17.3 MB of packed weights resident: twice the Infinity Cache


def onebit_gemv_bytes(kind, M, N, K):
    """Algorithmic bytes of one 1-bit-activation GEMV: packed weights (1 or 2 bits), the
    activation bits, fp32 y written, the scales read."""
    return N * K // (8 if kind == "binary" else 4) + M * K // 8 + 4 * M * N + 4 + 4 * M


def run_onebit(args):
    """The bit-floor page's GEMV shapes against binarized tokens: per copy, one
    bt_binarize_act per layout and the three GEMVs (bt_binary_gemv for the binary matrix,
    bt_ternary_gemv_a1 for the two ternary ones), replayed as one HIP graph."""
    import torch

    import bit_ternary_weight_absmean_amd as bt
    from bit_ternary_weight_absmean_amd import synth

    dev = torch.device("cuda:0")
    M = args.m or 1
    shapes = synth.SHAPES_ONEBIT
    K = shapes[0][2]
    ws = torch.empty(max(bt.pack_workspace_bytes(max(n for _, n, _ in shapes), K), 8), dtype=torch.uint8,
                     device=dev)
    packed = []
    for c in range(ONEBIT_COPIES):
        row = []
        for j, (kind, N, _) in enumerate(shapes):
            W = synth.device_gaussian((N, K), synth.weight_seed(synth.CFG_ONEBIT, c, j), dev, std=synth.WEIGHT_STD)
            row.append(bt.pack_weights_binary(W, ws) if kind == "binary" else bt.pack_weights(W, ws))
            del W
        packed.append(row)
    X = torch.from_numpy(synth.layer_activation(synth.CFG_ONEBIT, 0, M, K)).to(dev)
    bp = bt.binarize_act(X, bt.BITS_PLAIN)
    bc = bt.binarize_act(X, bt.BITS_CODES)
    ys = [torch.empty((M, N), dtype=torch.float32, device=dev) for _, N, _ in shapes]
    torch.cuda.synchronize()

    def products():
        for row in packed:
            bt.binary_gemv(row[0], bp, out_y=ys[0])
            bt.ternary_gemv_a1(row[1], bc, out_y=ys[1])
            bt.ternary_gemv_a1(row[2], bc, out_y=ys[2])

    def step():
        for row in packed:
            bt.binarize_act(X, bt.BITS_PLAIN, out=bp)
            bt.binary_gemv(row[0], bp, out_y=ys[0])
            bt.binarize_act(X, bt.BITS_CODES, out=bc)
            bt.ternary_gemv_a1(row[1], bc, out_y=ys[1])
            bt.ternary_gemv_a1(row[2], bc, out_y=ys[2])

    stream = torch.cuda.Stream(device=dev)

    def timed(fn):
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            fn()
        stream.synchronize()
        for _ in range(args.warmup):
            graph.replay()
        stream.synchronize()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record(stream)
        for _ in range(args.steps):
            graph.replay()
        end.record(stream)
        end.synchronize()
        return start.elapsed_time(end) / args.steps

    with torch.cuda.stream(stream):
        step()
        stream.synchronize()
        ms_step = timed(step)
        ms_prod = timed(products)
    prod_bytes = ONEBIT_COPIES * sum(onebit_gemv_bytes(kind, M, N, K) for kind, N, _ in shapes)
    step_bytes = prod_bytes + ONEBIT_COPIES * 2 * (4 * M * K + M * K // 8 + 4 * M)
    ops = ONEBIT_COPIES * sum(2 * M * N * K for _, N, _ in shapes)
    n_prod = ONEBIT_COPIES * len(shapes)
    prod_us = ms_prod * 1e3 / n_prod
    ach = prod_bytes / n_prod / (prod_us * 1e-6) / 1e9
    cpu = None if args.no_cpu_baseline else run_onebit_cpu_baseline(args, M)
    line = {
        "metric": METRIC,
        "value": round(step_bytes / (ms_step * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u32",
        "data": "synthetic",
        "config": {"workload": f"bit-floor GEMV shapes against binarized tokens (M={M}): 4096x4096 binary "
                               f"(bt_binary_gemv), 4096x4096 and 11008x4096 ternary (bt_ternary_gemv_a1); "
                               f"{ONEBIT_COPIES} copies resident", "M": M,
                   "launch": "hipGraph",
                   "step": "per copy: bt_binarize_act x 2 layouts + the three GEMVs"},
        "roofline": {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": None},
        "cpu_baseline": cpu,
        "detail": {"dominant_kernel": "k_gemv_bits", "kernel_avg_us": round(prod_us, 3),
                   "algorithmic_bytes_per_launch": round(prod_bytes / n_prod),
                   "gemv_GOPS": round(ops / (ms_prod * 1e-3) / 1e9, 1),
                   "resident_packed_bytes": sum(p.data.numel() for row in packed for p in row)},
    }
    print(json.dumps(line), flush=True)
    return 0


def run_onebit_cpu_baseline(args, M):
    """The oracle's W1A1 and W1.58A1 layers on copy 0's three matrices, single-threaded,
    repeated for about --cpu-seconds."""
    import oracle
    from bit_ternary_weight_absmean_amd import synth

    lib = oracle.load()
    K = synth.SHAPES_ONEBIT[0][2]
    X = synth.layer_activation(synth.CFG_ONEBIT, 0, M, K)
    mats = [(kind, synth.layer_weight(synth.CFG_ONEBIT, 0, j, N, K)) for j, (kind, N, _) in
            enumerate(synth.SHAPES_ONEBIT)]
    done = passes = 0
    t0 = time.perf_counter()
    while True:
        for kind, W in mats:
            (oracle.binary_layer if kind == "binary" else oracle.ternary_a1_layer)(W, X, lib)
            done += onebit_gemv_bytes(kind, M, W.shape[0], K)
        passes += 1
        el = time.perf_counter() - t0
        if el >= args.cpu_seconds:
            break
    return {"value": round(done / el / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"copy 0's three matrices at M={M} (weights packed in the timed loop), {passes} passes"}


# ----------------------------------------------------------- CPU baseline leg
def run_cpu_baseline(args, spec):
    """The oracle as it stands, single-threaded, on a bounded sample of the same workload:
    layer 0's matrices (all four shapes; for prefill the first 16 tokens), repeated until
    about --cpu-seconds of CPU work."""
    import oracle
    from bit_ternary_weight_absmean_amd import synth

    M = spec["M"] if not spec["prefill"] else min(spec["M"], 16)
    cfg = spec["cfg"]
    lib = oracle.load()
    mats = []
    for j, (_, N, K) in enumerate(spec["shapes"]):
        W = synth.layer_weight(cfg, 0, j, N, K)
        g = oracle.absmean(W, lib)
        mats.append((oracle.ternarize(W, g, lib), g, synth.layer_activation(cfg, j, M, K)))
        del W
    done_bytes = done_ops = passes = 0
    t0 = time.perf_counter()
    while True:
        for T, g, X in mats:
            Q, s, qs = oracle.quant_act(X, lib)
            acc = oracle.ternary_matmul(T, Q, lib)
            oracle.scale_epilogue(acc, g, s, lib)
            N, K = T.shape
            done_bytes += linear_bytes(M, N, K)
            done_ops += 2 * M * N * K
        passes += 1
        el = time.perf_counter() - t0
        if el >= args.cpu_seconds:
            break
    if spec["prefill"]:
        value, unit = done_ops / el / 1e12, "TOPS"
    else:
        value, unit = done_bytes / el / 1e9, "GB/s"
    return {"value": round(value, 4), "unit": unit, "cores": 1, "kind": "oracle",
            "sample": f"layer 0 of the workload ({len(mats)} matrices, M={M}), {passes} pass(es) in {el:.1f} s "
                      "of the single-threaded C oracle (quantize + int32 triple loop + epilogue), bytes and ops "
                      "counted as for the GPU step"}


# ----------------------------------------------------------- counters
def calib_copy():
    import torch

    n = 1 << 28  # 1 GiB of fp32
    a = torch.ones(n, dtype=torch.float32, device="cuda:0")
    b = torch.empty_like(a)
    for _ in range(10):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"calib_copy_bytes_each_way": 4 * n, "copies": 10}))


def _pmc_rows(d, counter):
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    rows = []
    for f in files:
        with open(f) as fh:
            rows += [r for r in csv.DictReader(fh) if r.get("Counter_Name") == counter]
    return rows


def summarize_pmc(args):
    fetch_dir, write_dir, cal_fetch_dir, cal_write_dir, out_json = args.summarize_pmc
    spec = workload_spec(args.workload, args.m)
    if args.split:
        kernel = "k_gemm" if spec["prefill"] else "k_gemv_direct"
    else:
        kernel = "k_gemm" if spec["prefill"] else "k_linear_decode"

    def per_launch_kib(d, counter, match):
        vals = [float(r["Counter_Value"]) for r in _pmc_rows(d, counter) if match(r["Kernel_Name"])]
        if not vals:
            raise SystemExit(f"no {counter} rows for the kernel in {d}")
        return sum(vals) / len(vals), len(vals)

    def is_kernel(name):
        return kernel in name

    def is_copy(name):
        return ("copy" in name.lower() or "elementwise" in name.lower()) and "bt::" not in name

    fetch_kib, n_f = per_launch_kib(fetch_dir, "FETCH_SIZE", is_kernel)
    write_kib, n_w = per_launch_kib(write_dir, "WRITE_SIZE", is_kernel)
    cal_fetch_kib, _ = per_launch_kib(cal_fetch_dir, "FETCH_SIZE", is_copy)
    cal_write_kib, _ = per_launch_kib(cal_write_dir, "WRITE_SIZE", is_copy)
    copy_bytes = 4 * (1 << 28)
    f_fetch = copy_bytes / (cal_fetch_kib * 1024)
    f_write = copy_bytes / (cal_write_kib * 1024)
    M = spec["M"]
    alg = [linear_bytes(M, N, K) if kernel == "k_linear_decode" else gemv_bytes(M, N, K)
           for _, N, K in spec["shapes"]]
    out = {
        "kernel": kernel, "workload": spec["desc"], "M": M,
        "source_sha256": source_hash(kernel),
        "launches_counted": {"FETCH_SIZE": n_f, "WRITE_SIZE": n_w},
        "fetch_kib_per_launch_raw": round(fetch_kib, 1), "write_kib_per_launch_raw": round(write_kib, 1),
        "copy_calibration": {"bytes_each_way": copy_bytes, "FETCH_SIZE_kib": round(cal_fetch_kib, 1),
                             "WRITE_SIZE_kib": round(cal_write_kib, 1), "fetch_factor": round(f_fetch, 4),
                             "write_factor": round(f_write, 4)},
        "traffic_bytes_per_launch": round(fetch_kib * 1024 * f_fetch + write_kib * 1024 * f_write),
        "algorithmic_bytes_per_launch": round(sum(alg) / len(alg)),
        "command": args.command,
    }
    with open(out_json, "w") as fh:
        json.dump(out, fh, indent=1)
        fh.write("\n")
    print(json.dumps(out))


def summarize_mfma(args):
    """Per-dispatch MFMA utilization of k_gemm: rocprofv3's MfmaUtil (MFMA-busy cycles of all SIMDs over
    GPU-active cycles times the SIMD count, i.e. measured at the clock the chip actually ran) and the int8
    MFMA op count (SQ_INSTS_VALU_MFMA_MOPS_I8, units of 512 ops) against the algorithmic 2*M*N*K."""
    pmc_dir, out_json = args.summarize_mfma
    spec = workload_spec(args.workload, args.m)
    if not spec["prefill"]:
        raise SystemExit("--summarize-mfma is for the prefill workload")
    kernel = "k_gemm"
    util = [float(r["Counter_Value"]) for r in _pmc_rows(pmc_dir, "MfmaUtil") if kernel in r["Kernel_Name"]]
    mops = [float(r["Counter_Value"]) for r in _pmc_rows(pmc_dir, "SQ_INSTS_VALU_MFMA_MOPS_I8")
            if kernel in r["Kernel_Name"]]
    if not util or not mops:
        raise SystemExit(f"no MfmaUtil / SQ_INSTS_VALU_MFMA_MOPS_I8 rows for {kernel} in {pmc_dir}")
    M = spec["M"]
    alg_ops = [2 * M * N * K for _, N, K in spec["shapes"]]
    # per matrix shape (identified by its exact op count), with the dispatch durations of the
    # counter run itself
    shape_of = {2 * M * N * K: f"{n} {N}x{K}" for n, N, K in spec["shapes"]}
    per = collections.defaultdict(lambda: {"util": [], "ops": [], "us": []})
    util_rows = [r for r in _pmc_rows(pmc_dir, "MfmaUtil") if kernel in r["Kernel_Name"]]
    mops_rows = {r["Dispatch_Id"]: float(r["Counter_Value"]) for r in _pmc_rows(pmc_dir, "SQ_INSTS_VALU_MFMA_MOPS_I8")
                 if kernel in r["Kernel_Name"]}
    for r in util_rows:
        ops = 512 * mops_rows.get(r["Dispatch_Id"], 0.0)
        key = shape_of.get(round(ops), f"grid {r['Grid_Size']}")
        per[key]["util"].append(float(r["Counter_Value"]))
        per[key]["ops"].append(ops)
        per[key]["us"].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    per_shape = {k: {"launches": len(v["util"]), "mfma_util_percent": round(sum(v["util"]) / len(v["util"]), 2),
                     "dispatch_us_under_counters": round(sum(v["us"]) / len(v["us"]), 2),
                     "TOPS_under_counters": round(sum(v["ops"]) / sum(v["us"]) / 1e6, 1)}
                 for k, v in per.items()}
    out = {
        "kernel": kernel, "workload": spec["desc"], "M": M,
        "source_sha256": source_hash(kernel),
        "launches_counted": len(util),
        "per_shape": per_shape,
        "mfma_util_percent_mean": round(sum(util) / len(util), 2),
        "mfma_util_percent_min": round(min(util), 2), "mfma_util_percent_max": round(max(util), 2),
        "int8_mfma_ops_per_launch": round(512 * sum(mops) / len(mops)),
        "algorithmic_ops_per_launch": round(sum(alg_ops) / len(alg_ops)),
        "command": args.command,
    }
    with open(out_json, "w") as fh:
        json.dump(out, fh, indent=1)
        fh.write("\n")
    print(json.dumps(out))


def mfma_util_for(spec, kernel):
    """Mean MfmaUtil (%) from the committed counter summary, while the kernel sources still match."""
    if ROW_SCALES:
        return None  # the committed counters were taken with one scale per matrix
    path = os.path.join(ROOT, "profiles", f"mfma_{kernel}_{spec['name']}_m{spec['M']}.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("source_sha256") != source_hash(kernel):
        return None
    return rec["mfma_util_percent_mean"]


def traffic_for(spec, kernel):
    if ROW_SCALES:
        return None  # the committed counters were taken with one scale per matrix
    path = traffic_path(spec["name"], kernel, spec["M"])
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("source_sha256") != source_hash(kernel):
        return None  # the kernel changed since the counters were taken
    return rec["traffic_bytes_per_launch"]


# ----------------------------------------------------------------- entry
def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(the hot path is a single-GPU kernel; multi-GPU sharding is a design note only).",
              file=sys.stderr)
        return 2
    if args.summarize_pmc:
        summarize_pmc(args)
        return 0
    if args.summarize_mfma:
        summarize_mfma(args)
        return 0
    if args.calib_copy:
        calib_copy()
        return 0
    global ROW_SCALES
    ROW_SCALES = args.row_scales
    if args.workload == "onebit_decode":
        return run_onebit(args)
    spec = workload_spec(args.workload, args.m)
    if ROW_SCALES:
        spec["desc"] += ", row-group weight scales (one per Q, K, V and gate, up block)"
    g = run_gpu(args, spec)
    M = spec["M"]
    prod_us = g["ms_prod"] * 1e3 / g["n_prod"]
    bytes_per_launch = g["prod_bytes"] / g["n_prod"]
    ops_per_launch = g["step_ops"] / g["n_prod"]
    traffic = traffic_for(spec, g["kernel"])
    if spec["prefill"]:
        value = g["step_ops"] / (g["ms_step"] * 1e-3) / 1e12
        unit = "TOPS"
        ach = ops_per_launch / (prod_us * 1e-6) / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 1), "peak": INT8_PEAK_TOPS, "unit": "TFLOP/s",
                "frac": round(ach / INT8_PEAK_TOPS, 4), "traffic": traffic}
    else:
        value = g["step_bytes"] / (g["ms_step"] * 1e-3) / 1e9
        unit = "GB/s"
        ach = bytes_per_launch / (prod_us * 1e-6) / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": traffic}
    cpu = None if args.no_cpu_baseline else run_cpu_baseline(args, spec)
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(g["ms_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": spec["desc"], "M": M, "layers": spec["layers"],
                   "shapes": [f"{n} {N}x{K}" for n, N, K in spec["shapes"]],
                   "resident_packed_bytes": g["resident"], "launch": g["launch"],
                   "step": ("per matrix: bt_ternary_linear (quantizer fused into the decode kernel)" if g["fused"]
                            else ("per matrix: bt_quant_act + " if args.split else
                                  "per matrix: bt_ternary_linear = bt_quant_act + ") +
                            ("bt_ternary_gemm_ws" if g["kernel"] == "k_gemm" else "bt_ternary_gemv"))},
        "roofline": roof,
        "cpu_baseline": cpu,
        "detail": {"dominant_kernel": g["kernel"], "kernel_avg_us": round(prod_us, 3),
                   "algorithmic_bytes_per_launch": round(bytes_per_launch),
                   "ops_per_launch": round(ops_per_launch),
                   "step_hbm_frac": None if spec["prefill"] else round(value / HBM_PEAK_GBS, 4),
                   "step_TOPS": round(g["step_ops"] / (g["ms_step"] * 1e-3) / 1e12, 3),
                   "weights_per_s": round(sum(N * K for _, N, K in spec["shapes"]) * spec["layers"] /
                                          (g["ms_step"] * 1e-3), 1),
                   "setup_s": round(g["setup_s"], 1),
                   "mfma_util_percent_counters": mfma_util_for(spec, g["kernel"]) if spec["prefill"] else None},
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
