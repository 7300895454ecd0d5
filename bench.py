"""Benchmark of the W1.58A8 ternary linear layer hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--eager] [--no-cpu-baseline]

A step is one pass of the whole per-call hot path over one batch of synthetic input:
for every resident weight matrix, quantize its fp32 activations per token to int8, run
the integer ternary product and apply the scale epilogue -- one bt_ternary_linear call
per matrix (a single fused kernel at decode sizes; bt_quant_act + bt_ternary_gemm for
prefill). ``--split`` times the unfused route (bt_quant_act + bt_ternary_gemv/gemm as
two launches) instead. Weight packing is offline and outside the timed region. Inputs
are resident in HBM before timing starts. Prints ONE JSON line (one GPU).

Workloads (``--workload``):
  2b_decode   (default) 2B-class decode, M = 1: 30 layers x {QKV 3840x2560, O 2560x2560,
              gate+up 13824x2560, down 2560x6912}, all 120 packed matrices resident
              (521 MB, twice the 256 MB Infinity Cache) -> metric in GB/s.
  7b_decode   7B-class decode at --m (1, 4, 8): 32 layers of {12288x4096, 4096x4096,
              22016x4096, 4096x11008} resident (1.62 GB) -> GB/s.
  100b_decode 100B-class single-layer sweep at --m (1, 16): 3 independently seeded copies
              of {10240x8192, 8192x8192, 57344x8192, 8192x28672} (642 MB) -> GB/s.
  2b_prefill  2B-class prefill at --m (256, 2048): the 2B layer shapes, 30 layers -> TOPS.
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

METRIC = "ternary GEMV HBM GB/s (% of peak) at 2B decode shapes; prefill GEMM int8 TOPS"
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, 8 TB/s
INT8_PEAK_TOPS = 5000.0  # MI355X dense int8 MFMA, 5.0 POP/s


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="2b_decode", choices=["2b_decode", "7b_decode", "100b_decode", "2b_prefill"])
    p.add_argument("--m", type=int, default=None, help="tokens per call (default: 1 for decode, 2048 for prefill)")
    p.add_argument("--eager", action="store_true", help="launch kernels one by one instead of replaying a graph")
    p.add_argument("--split", action="store_true", help="time bt_quant_act + product as two launches per matrix")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=10.0, help="target CPU time of the oracle baseline")
    p.add_argument("--calib-copy", action="store_true",
                   help="only run a plain 1 GiB device copy 10 times (HBM counter calibration)")
    return p.parse_args()


# ----------------------------------------------------------------- workloads
def workload_spec(name, m):
    from bit_ternary_weight_absmean_amd import synth

    if name == "2b_decode":
        return dict(cfg=synth.CFG_2B_DECODE, shapes=synth.SHAPES_2B, layers=30, M=m or 1, prefill=False,
                    desc="2B-class decode GEMVs, 30 layers resident")
    if name == "7b_decode":
        return dict(cfg=synth.CFG_7B_DECODE, shapes=synth.SHAPES_7B, layers=32, M=m or 1, prefill=False,
                    desc="7B-class decode GEMVs, 32 layers resident")
    if name == "100b_decode":
        return dict(cfg=synth.CFG_100B_DECODE, shapes=synth.SHAPES_100B, layers=3, M=m or 1, prefill=False,
                    desc="100B-class single-layer decode sweep, 3 seeded copies resident")
    return dict(cfg=synth.CFG_2B_PREFILL, shapes=synth.SHAPES_2B, layers=30, M=m or 2048, prefill=True,
                desc="2B-class prefill GEMMs, 30 layers resident")


def gemv_bytes(M, N, K):
    """Algorithmic HBM bytes of one product call: 2-bit weights, int8 activations read,
    fp32 output written, gamma + s_x + sum q read."""
    return N * K // 4 + M * K + 4 * M * N + 4 + 8 * M


def linear_bytes(M, N, K):
    """Algorithmic HBM bytes of one fused decode call: 2-bit weights and fp32 activations
    read, fp32 output written, gamma read."""
    return N * K // 4 + 4 * M * K + 4 * M * N + 4


def quant_bytes(M, K):
    """Algorithmic bytes of one activation quantization: fp32 read, int8 + s_x + sum q written."""
    return 4 * M * K + M * K + 8 * M


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
        for j, (_, N, K) in enumerate(shapes):
            W = synth.device_gaussian((N, K), synth.weight_seed(cfg, layer, j), dev, std=synth.WEIGHT_STD)
            row.append(bt.pack_weights(W, workspace=ws))
            del W
        packed.append(row)
    torch.cuda.synchronize()
    setup_s = time.time() - t0
    resident = sum(p.data.numel() for row in packed for p in row)

    # Per-matrix-type activations, output buffers and (route permitting) workspaces.
    xs, qs, ys, wss = [], [], [], []
    for j, (_, N, K) in enumerate(shapes):
        X = torch.from_numpy(synth.layer_activation(cfg, j, M, K)).to(dev)
        xs.append(X)
        qs.append(bt.quant_act(X))
        ys.append(torch.empty((M, N), dtype=torch.float32, device=dev))
        wb = bt.linear_workspace_bytes(M, N, K)
        wss.append(torch.empty(wb, dtype=torch.uint8, device=dev) if wb else None)
    torch.cuda.synchronize()

    product = bt.ternary_gemm if spec["prefill"] else bt.ternary_gemv

    if args.split:
        def call(j, pw):
            bt.quant_act(xs[j], out=qs[j])
            product(pw, qs[j], out_y=ys[j])
    else:
        def call(j, pw):
            bt.linear(xs[j], pw, out_y=ys[j], workspace=wss[j])

    def step():
        for row in packed:
            for j, pw in enumerate(row):
                call(j, pw)

    stream = torch.cuda.Stream(device=dev)
    graph = None
    with torch.cuda.stream(stream):
        for _ in range(2):
            step()
        stream.synchronize()
        if not args.eager:
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph, stream=stream):
                step()
            stream.synchronize()

        run = graph.replay if graph is not None else step
        for _ in range(args.warmup):
            run()
        stream.synchronize()
        torch.cuda.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record(stream)
        for _ in range(args.steps):
            run()
        end.record(stream)
        end.synchronize()
        torch.cuda.synchronize()
        ms_step = start.elapsed_time(end) / args.steps

        # Dominant kernel (the product, with the quantizer fused in at decode sizes) timed
        # live: one event pair around every product launch, eager, on the kernels' stream.
        per_shape_ms = [0.0] * len(shapes)
        reps = max(2, min(args.steps, 5))
        pairs = []
        fused = not args.split and not spec["prefill"]
        for _ in range(reps):
            for row in packed:
                for j, pw in enumerate(row):
                    if not fused:
                        bt.quant_act(xs[j], out=qs[j])
                    e0 = torch.cuda.Event(enable_timing=True)
                    e1 = torch.cuda.Event(enable_timing=True)
                    e0.record(stream)
                    if fused:
                        bt.linear(xs[j], pw, out_y=ys[j], workspace=wss[j])
                    else:
                        product(pw, qs[j], out_y=ys[j])
                    e1.record(stream)
                    pairs.append((j, e0, e1))
        stream.synchronize()
    for j, e0, e1 in pairs:
        per_shape_ms[j] += e0.elapsed_time(e1)
    n_per_shape = reps * spec["layers"]
    per_shape_us = [1e3 * t / n_per_shape for t in per_shape_ms]

    step_bytes = 0
    step_ops = 0
    prod_bytes = 0
    fused = not args.split and not spec["prefill"]
    for row in packed:
        for j, (_, N, K) in enumerate(shapes):
            # the fused kernel reads fp32 x once and never writes or re-reads int8 Xq
            step_bytes += linear_bytes(M, N, K) if fused else gemv_bytes(M, N, K) + quant_bytes(M, K)
            prod_bytes += linear_bytes(M, N, K) if fused else gemv_bytes(M, N, K)
            step_ops += 2 * M * N * K
    n_prod = spec["layers"] * len(shapes)
    prod_us_avg = sum(per_shape_us) / len(shapes)
    detail = []
    for j, (name, N, K) in enumerate(shapes):
        b = linear_bytes(M, N, K) if fused else gemv_bytes(M, N, K)
        detail.append({"shape": name, "N": N, "K": K, "us": round(per_shape_us[j], 3),
                       "GB/s": round(b / (per_shape_us[j] * 1e3), 1),
                       "TOPS": round(2 * M * N * K / (per_shape_us[j] * 1e6), 2)})
    return dict(ms_step=ms_step, step_bytes=step_bytes, step_ops=step_ops, prod_bytes=prod_bytes,
                n_prod=n_prod, prod_us_avg=prod_us_avg, detail=detail, resident=resident, setup_s=setup_s,
                launch="hipGraph" if graph is not None else "eager", fused=fused)


# ----------------------------------------------------------- CPU baseline leg
def run_cpu_baseline(args, spec):
    """The oracle as it stands, single-threaded, on a bounded sample of the same workload:
    layer 0's matrices (all four shapes), repeated until about --cpu-seconds of CPU work."""
    import oracle
    from bit_ternary_weight_absmean_amd import synth

    M = spec["M"]
    cfg = spec["cfg"]
    lib = oracle.load()
    mats = []
    for j, (_, N, K) in enumerate(spec["shapes"]):
        W = synth.layer_weight(cfg, 0, j, N, K)
        g = oracle.absmean(W, lib)
        mats.append((oracle.ternarize(W, g, lib), g, synth.layer_activation(cfg, j, M, K)))
        del W
    done_bytes = 0
    done_ops = 0
    passes = 0
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
        if el >= args.cpu_seconds or (spec["prefill"] and passes >= 1):
            break
    value = done_bytes / el / 1e9 if not spec["prefill"] else done_ops / el / 1e12
    unit = "GB/s" if not spec["prefill"] else "TOPS"
    return {"value": round(value, 4), "unit": unit, "cores": 1, "kind": "oracle",
            "sample": f"layer 0 of the workload ({len(mats)} matrices, M={M}), {passes} pass(es), "
                      f"{el:.1f} s single-threaded C oracle (quantize + int32 triple loop + epilogue)"}


def calib_copy():
    import torch

    n = 1 << 28  # 1 GiB of fp32
    a = torch.ones(n, dtype=torch.float32, device="cuda:0")
    b = torch.empty_like(a)
    for _ in range(10):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"calib_copy_bytes_each_way": 4 * n, "copies": 10}))


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(the hot path is a single-GPU kernel; multi-GPU sharding is a design note only).",
              file=sys.stderr)
        return 2
    if args.calib_copy:
        calib_copy()
        return 0
    spec = workload_spec(args.workload, args.m)
    g = run_gpu(args, spec)
    M = spec["M"]
    if spec["prefill"]:
        value = g["step_ops"] / (g["ms_step"] * 1e-3) / 1e12
        unit = "TOPS"
        ach = g["step_ops"] / spec["layers"] / len(spec["shapes"]) / (g["prod_us_avg"] * 1e-6) / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 1), "peak": INT8_PEAK_TOPS, "unit": "TFLOP/s",
                "frac": round(ach / INT8_PEAK_TOPS, 4), "traffic": None}
    else:
        value = g["step_bytes"] / (g["ms_step"] * 1e-3) / 1e9
        unit = "GB/s"
        ach = g["prod_bytes"] / g["n_prod"] / (g["prod_us_avg"] * 1e-6) / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": None}
    cpu = None
    if not args.no_cpu_baseline:
        cpu = run_cpu_baseline(args, spec)
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
                            else "per matrix: bt_quant_act + " +
                            ("bt_ternary_gemm" if spec["prefill"] else "bt_ternary_gemv"))},
        "roofline": roof,
        "cpu_baseline": cpu,
        "detail": {"hbm_frac_of_step": round(value / HBM_PEAK_GBS, 4) if not spec["prefill"] else None,
                   "weights_per_s": round(sum(N * K for _, N, K in spec["shapes"]) * spec["layers"] /
                                          (g["ms_step"] * 1e-3), 1),
                   "step_TOPS": round(g["step_ops"] / (g["ms_step"] * 1e-3) / 1e12, 3),
                   "product_kernel_avg_us": round(g["prod_us_avg"], 3),
                   "per_shape": g["detail"], "setup_s": round(g["setup_s"], 1)},
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
