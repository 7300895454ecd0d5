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
    "k_gemv_blocked": ["decode.hip", "wave.h", "bt_internal.h"],
    "k_gemv_dot4": ["gemv.hip", "bt_internal.h"],
    "k_gemv_lut": ["lut.hip", "bt_internal.h"],
    "k_gemm": ["gemm.hip", "bt_internal.h"],
    "k_gemm_ks": ["gemm.hip", "bt_internal.h"],
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
    p.add_argument("--no-ceilings", action="store_true",
                   help="skip the achievable-ceiling kernels (launch floor, plain reads, MFMA loop)")
    p.add_argument("--no-prefill", action="store_true",
                   help="2b_decode only: skip the prefill half of the metric (2B prefill GEMM at M = 2048)")
    p.add_argument("--no-workloads", action="store_true",
                   help="2b_decode only: skip the other configurations (detail.workloads: 2B decode at 4 tokens, "
                        "7B decode at 1, 4, 8, 2B prefill at 256, 100B decode at 1, 16)")
    p.add_argument("--cpu-cores", type=int, default=None,
                   help="worker processes of the all-cores oracle baseline (default: the usable cores, at most 16)")
    p.add_argument("--summarize-trace", nargs=2, metavar=("TRACE_DIR[,TRACE_DIR...]", "OUT_MD"),
                   help="write a per-kernel summary (durations and launch intervals) of a rocprofv3 --kernel-trace "
                        "--stats run of this workload")
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
    p.add_argument("--summarize-sq", nargs=3, metavar=("PASS1_DIR", "PASS2_DIR", "OUT_MD"),
                   help="write the prefill GEMM's per-shape wave-time breakdown from the two rocprofv3 --pmc "
                        "passes of SQ counters listed in SQ_PASSES, run on this workload")
    p.add_argument("--command", default="", help="the rocprofv3 command line recorded with --summarize-pmc / -mfma")
    return p.parse_args()


# ----------------------------------------------------------------- workloads
# Token counts each workload is measured at (``--m``). tests/test_plan_coverage.py checks that
# every kernel instance these steps launch -- default, --split and --row-scales routes -- is
# also run by a parity test against the oracle.
WORKLOAD_M = {"2b_decode": (1, 4), "7b_decode": (1, 2, 4, 8), "100b_decode": (1, 2, 4, 16), "2b_prefill": (256, 2048)}


def step_plans(spec, split=False, row_scales=False, gemv_algo="auto"):
    """The kernel instances (bt_kernel_plan text) one step of ``spec`` launches, per matrix."""
    import bit_ternary_weight_absmean_amd as bt

    M = spec["M"]
    algo = {"auto": bt.GEMV_AUTO, "mfma": bt.GEMV_MFMA, "staged": bt.GEMV_STAGED, "dot4": bt.GEMV_DOT4,
            "lut": bt.GEMV_LUT}[gemv_algo]
    plans = []
    for _, N, K in spec["shapes"]:
        if not split:
            plans.append(bt.kernel_plan(bt.CALL_LINEAR, M, N, K, row_scales=row_scales))
        elif spec["prefill"] or M > bt.GEMV_MAX_M:
            plans.append(bt.kernel_plan(bt.CALL_QUANT, M, N, K) + " + " +
                         bt.kernel_plan(bt.CALL_GEMM_WS, M, N, K, row_scales=row_scales))
        else:
            plans.append(bt.kernel_plan(bt.CALL_QUANT, M, N, K) + " + " +
                         bt.kernel_plan(bt.CALL_GEMV, M, N, K, algo, row_scales=row_scales))
    return plans


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

    # Route of each matrix shape, as the step runs it: the fused decode kernel where
    # bt_ternary_linear takes it (no workspace), else the product kernel on activations the
    # quantizer launch wrote (--split: always the latter).
    fused_j = [(not args.split) and bt.linear_workspace_bytes(M, N, K) == 0 for _, N, K in shapes]
    fused = all(fused_j)
    gemm = spec["prefill"] or M > bt.GEMV_MAX_M
    names = {"mfma": "k_gemv_direct", "staged": "k_gemv_staged", "dot4": "k_gemv_dot4", "lut": "k_gemv_lut"}

    def staged_name(N, K):  # whole rows in LDS, or rows staged in K-blocks
        return "k_gemv_staged" if M * ((K + 255) // 256 * 256) <= 131072 else "k_gemv_blocked"

    def kernel_of(j):
        _, N, K = shapes[j]
        if fused_j[j]:
            return "k_linear_decode"
        if gemm:  # the small-M form where the GEMM takes it (few tiles), else k_gemm
            small = bt.kernel_plan(bt.CALL_GEMM_WS, M, N, K).startswith("k_gemm_ks")
            return "k_gemm_ks" if small else "k_gemm"
        if args.gemv_algo in ("auto", "staged"):  # BT_GEMV_AUTO takes the staged forms, as bt_ternary_linear
            return staged_name(N, K)
        return names[args.gemv_algo]
    kernel = " + ".join(dict.fromkeys(kernel_of(j) for j in range(len(shapes))))
    algo = {"auto": bt.GEMV_AUTO, "mfma": bt.GEMV_MFMA, "staged": bt.GEMV_STAGED, "dot4": bt.GEMV_DOT4,
            "lut": bt.GEMV_LUT}[args.gemv_algo]

    def product(pw, q, out_y, j):
        if gemm:
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
        """The product launches of one step: the fused kernel where the step runs it, else the
        product kernel on the already quantized activations (the quantizer launches left out)."""
        for row in packed:
            for j, pw in enumerate(row):
                if fused_j[j]:
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
        # per matrix shape, in the context of the step: the product graph's time minus that of
        # the same graph without the shape's launches, over the layers (a graph of one shape
        # alone would re-read a few matrices from the Infinity Cache and carry the replay's
        # fixed cost on few launches)
        shape_us = []
        for j in range(len(shapes)):
            def all_but(j=j):
                for row in packed:
                    for jj, pw in enumerate(row):
                        if jj == j:
                            continue
                        if fused_j[jj]:
                            bt.linear(xs[jj], pw, out_y=ys[jj])
                        else:
                            product(pw, qs[jj], ys[jj], jj)
            shape_us.append((ms_prod - timed(all_but, args.steps, args.warmup)) * 1e3 / spec["layers"])

    step_bytes = step_ops = prod_bytes = 0
    for row in packed:
        for j, (_, N, K) in enumerate(shapes):
            # the fused kernel reads fp32 x once and never writes or re-reads int8 Xq
            if fused_j[j]:
                step_bytes += linear_bytes(M, N, K)
                prod_bytes += linear_bytes(M, N, K)
            else:
                step_bytes += gemv_bytes(M, N, K) + quant_bytes(M, K)
                prod_bytes += gemv_bytes(M, N, K)
            step_ops += 2 * M * N * K
    n_prod = spec["layers"] * len(shapes)
    return dict(ms_step=ms_step, ms_prod=ms_prod, step_bytes=step_bytes, step_ops=step_ops,
                prod_bytes=prod_bytes, n_prod=n_prod, resident=resident, setup_s=setup_s,
                launch="eager" if args.eager else "hipGraph", fused=fused, fused_any=any(fused_j), kernel=kernel,
                shape_us=shape_us,
                packed=packed, stream=stream, timed=timed)


# ------------------------------------------------------- achievable ceilings
def ceilings_lib():
    """libbt_ceilings.so: the empty-launch, plain-read and MFMA-loop kernels (built with libbt.so)."""
    import ctypes

    path = os.path.join(ROOT, "bit_ternary_weight_absmean_amd", "libbt_ceilings.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: run `python -m bit_ternary_weight_absmean_amd.build`")
    L = ctypes.CDLL(path)
    i32, i64, vp, u32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_uint32
    L.btc_launch_empty.argtypes = [i32, i32, i32, vp, vp]
    L.btc_read_blocks.argtypes = [i64, i32]
    L.btc_launch_read.argtypes = [vp, i64, i32, vp, vp]
    L.btc_launch_mfma.argtypes = [i32, i32, u32, vp, vp]
    for f in (L.btc_launch_empty, L.btc_read_blocks, L.btc_launch_read, L.btc_launch_mfma):
        f.restype = i32
    return L


LARGE_READ_BYTES = 117_440_512  # the 100B-class gate+up matrix packed at 2 bits
MFMA_OPS = 2 * 16 * 16 * 64     # one v_mfma_i32_16x16x64_i8


def run_ceilings(args, spec, g):
    """What the hardware gives this workload with no method arithmetic: the launch floor of
    the step's graph, a plain read of each resident matrix in the step's launch structure,
    a plain read of a large matrix, and the int8 MFMA rate (bench.py --ceilings alone, or
    detail.ceilings of the default run)."""
    import torch

    L = ceilings_lib()
    stream, timed, packed = g["stream"], g["timed"], g["packed"]
    dev = torch.device("cuda:0")
    sink = torch.zeros(1 << 20, dtype=torch.int32, device=dev)
    out, s = sink.data_ptr(), stream.cuda_stream
    n_launch = g["n_prod"]
    steps, warmup = max(args.steps, 5), max(args.warmup, 2)

    def ok(rc):
        if rc != 0:
            raise RuntimeError(f"ceiling kernel launch failed (hipError {rc})")

    res = {}
    with torch.cuda.stream(stream):
        # launch floor: the graph of n_launch back-to-back launches, at the first matrix's grid
        _, N0, _ = spec["shapes"][0]
        grid0 = -(-N0 // 16)  # one workgroup per 16-row block at most: an upper bound on the fused grid
        for store in (0, 1):
            def empties(store=store):
                for _ in range(n_launch):
                    ok(L.btc_launch_empty(grid0, 512, store, out, s))
            res["launch_floor_store_us" if store else "launch_floor_us"] = round(
                timed(empties, steps, warmup) * 1e3 / n_launch, 3)
        # plain read of each resident matrix, one launch per matrix as in the step: the loads per
        # thread (1, 2, 4 or 8) that give the fastest read step, then each shape's time in that
        # step's context (the step's time minus that of the step without the shape's reads)
        def read_step(us_of=None, skip=None):
            for row in packed:
                for j, pw in enumerate(row):
                    if j != skip:
                        ok(L.btc_launch_read(pw.data.data_ptr(), pw.data.numel(), us_of[j], out, s))
        nshape = len(spec["shapes"])
        best_u = [1] * nshape
        for j in range(nshape):
            best = None
            for u in (1, 2, 4, 8):
                trial = list(best_u)
                trial[j] = u
                ms = timed(lambda: read_step(trial), steps, warmup)
                if best is None or ms < best[0]:
                    best = (ms, u)
            best_u[j] = best[1]
        read_ms = timed(lambda: read_step(best_u), steps, warmup)
        per_shape = {}
        for j, (name, N, K) in enumerate(spec["shapes"]):
            nbytes = packed[0][j].data.numel()
            us = (read_ms - timed(lambda: read_step(best_u, j), steps, warmup)) * 1e3 / len(packed)
            per_shape[name] = {"bytes": nbytes, "read_us": round(us, 3), "read_GBs": round(nbytes / (us * 1e-6) / 1e9, 1),
                               "loads_per_thread": best_u[j], "product_us": round(g["shape_us"][j], 3),
                               "product_frac_of_read": round(us / g["shape_us"][j], 4)}
        res["per_shape"] = per_shape
        res["read_step_ms"] = round(read_ms, 5)
        read_bytes = sum(pw.data.numel() for row in packed for pw in row)
        res["read_step_GBs"] = round(read_bytes / (read_ms * 1e-3) / 1e9, 1)
        res["step_frac_of_read_step"] = round(read_ms / g["ms_step"], 4)
        # a large plain read (three rotating buffers, 352 MB: more than the 256 MB Infinity Cache)
        bufs = [torch.empty(LARGE_READ_BYTES, dtype=torch.uint8, device=dev) for _ in range(3)]
        for b in bufs:
            b.fill_(1)
        best = None
        for u in (2, 4, 8):
            def big(u=u):
                for _ in range(2):
                    for b in bufs:
                        ok(L.btc_launch_read(b.data_ptr(), LARGE_READ_BYTES, u, out, s))
            us = timed(big, steps, warmup) * 1e3 / 6
            best = us if best is None else min(best, us)
        res["large_read"] = {"bytes": LARGE_READ_BYTES, "us": round(best, 2),
                             "GBs": round(LARGE_READ_BYTES / (best * 1e-6) / 1e9, 1)}
        del bufs
        # int8 MFMA loop at one to three waves per SIMD
        iters = 4000
        mf = {}
        for wps in (1, 2, 3, 4):
            blocks = 256 * wps

            def loop(blocks=blocks):
                ok(L.btc_launch_mfma(blocks, iters, 12345, out, s))
            ms = timed(loop, 5, 2)
            mf[wps] = blocks * 4 * iters * 16 * MFMA_OPS / (ms * 1e-3) / 1e12
        wps = max(mf, key=mf.get)
        res["mfma_int8_TOPS"] = round(mf[wps], 1)
        res["mfma_waves_per_simd"] = wps
        res["mfma_int8_TOPS_by_waves_per_simd"] = {str(k): round(v, 1) for k, v in mf.items()}
        # a library dense int8 GEMM (torch._int_mm: hipBLASLt / rocBLAS) of the 2B prefill gate+up
        # shape on unpacked int8 operands, for reference
        try:
            A = torch.randint(-127, 128, (2048, 2560), dtype=torch.int8, device=dev)
            B = torch.randint(-1, 2, (13824, 2560), dtype=torch.int8, device=dev).t()
            torch._int_mm(A, B)
            torch.cuda.synchronize()
            ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            ev0.record(stream)
            for _ in range(20):
                torch._int_mm(A, B)
            ev1.record(stream)
            ev1.synchronize()
            ms = ev0.elapsed_time(ev1) / 20
            res["library_int8_gemm"] = {"shape": "2048 x 13824 x 2560 (torch._int_mm, int8 in, int32 out)",
                                        "us": round(ms * 1e3, 2),
                                        "TOPS": round(2 * 2048 * 13824 * 2560 / (ms * 1e-3) / 1e12, 1)}
            del A, B
        except Exception as e:  # reported, not fatal: the reference is optional
            res["library_int8_gemm"] = {"error": str(e)[:200]}
    torch.cuda.synchronize()
    return res


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
        "detail": {"dominant_kernel": "k_gemv_bits", "launch_interval_us": round(prod_us, 3),
                   "launch_interval_note": "the GEMV launches of one step replayed as a HIP graph (binarize "
                                           "launches left out), timed with HIP events, divided by the launches",
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
# Matrices of the CPU sample, inherited by the all-cores worker processes (fork).
_CPU_MATS = []


def _cpu_rows(task):
    """Worker of the all-cores baseline: the oracle's int32 triple loop on a block of
    output rows of one sample matrix."""
    import oracle

    i, r0, r1, Q = task
    T = _CPU_MATS[i][0]
    return i, r0, oracle.ternary_matmul(T[r0:r1], Q)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def usable_cores(limit=16):
    """Cores this process may run on, at most `limit` (the host share of one GPU)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, limit))


def run_cpu_baseline(args, spec):
    """The oracle as it stands, on a bounded sample of the same workload: layer 0's matrices
    (all four shapes; for prefill the first 16 tokens), repeated until about --cpu-seconds
    of work, first single-threaded, then with the int32 triple loop -- the dominant phase --
    spread over the usable cores in row blocks (worker processes calling the same oracle
    function; the results are identical, the sums being integer). Per-phase seconds are the
    totals over the passes: quantize (per-token absmax int8), the int32 loop, the epilogue;
    the offline weight scale + codes of each sample matrix are timed once."""
    import multiprocessing as mp

    import numpy as np

    import oracle
    from bit_ternary_weight_absmean_amd import synth

    global _CPU_MATS
    M = spec["M"] if not spec["prefill"] else min(spec["M"], 16)
    cfg = spec["cfg"]
    lib = oracle.load()
    mats = []
    t0 = time.perf_counter()
    for j, (_, N, K) in enumerate(spec["shapes"]):
        W = synth.layer_weight(cfg, 0, j, N, K)
        g = oracle.absmean(W, lib)
        mats.append((oracle.ternarize(W, g, lib), g, synth.layer_activation(cfg, j, M, K)))
        del W
    pack_s = time.perf_counter() - t0
    _CPU_MATS = mats
    pass_bytes = sum(linear_bytes(M, T.shape[0], T.shape[1]) for T, _, _ in mats)
    pass_ops = sum(2 * M * T.shape[0] * T.shape[1] for T, _, _ in mats)

    def run(pool, cores):
        ph = {"quantize": 0.0, "int32_loop": 0.0, "epilogue": 0.0}
        passes = 0
        accs = []
        t_start = time.perf_counter()
        while True:
            accs = []
            for i, (T, g, X) in enumerate(mats):
                t = time.perf_counter()
                Q, sx, _ = oracle.quant_act(X, lib)
                ph["quantize"] += time.perf_counter() - t
                t = time.perf_counter()
                if pool is None:
                    acc = oracle.ternary_matmul(T, Q, lib)
                else:
                    N = T.shape[0]
                    step = -(-N // cores)
                    acc = np.empty((M, N), np.int32)
                    for _, r0, part in pool.imap_unordered(_cpu_rows, [(i, r0, min(N, r0 + step), Q)
                                                                       for r0 in range(0, N, step)]):
                        acc[:, r0:r0 + part.shape[1]] = part
                ph["int32_loop"] += time.perf_counter() - t
                t = time.perf_counter()
                oracle.scale_epilogue(acc, g, sx, lib)
                ph["epilogue"] += time.perf_counter() - t
                accs.append(acc)
            passes += 1
            el = time.perf_counter() - t_start
            if el >= args.cpu_seconds / 2:
                break
        return passes, el, ph, accs

    p1, el1, ph1, acc1 = run(None, 1)
    cores = args.cpu_cores or usable_cores()
    ctx = mp.get_context("fork")
    with ctx.Pool(cores) as pool:
        pool.map(_cpu_rows, [(0, 0, 1, oracle.quant_act(mats[0][2], lib)[0])] * cores)  # start the workers
        pn, eln, phn, accn = run(pool, cores)
    _CPU_MATS = []
    for a, b in zip(acc1, accn):
        if not np.array_equal(a, b):
            raise RuntimeError("all-cores oracle baseline disagrees with the single-threaded one")

    def rate(passes, el):
        if spec["prefill"]:
            return passes * pass_ops / el / 1e12
        return passes * pass_bytes / el / 1e9

    unit = "TOPS" if spec["prefill"] else "GB/s"
    return {"value": round(rate(pn, eln), 4), "unit": unit, "cores": cores, "kind": "oracle",
            "sample": f"layer 0 of the workload ({len(mats)} matrices, M={M}) in passes of the C oracle "
                      f"(quantize + int32 triple loop + epilogue; bytes and ops counted as for the GPU step): "
                      f"{pn} passes in {eln:.1f} s with the int32 loop in row blocks over {cores} worker "
                      f"processes; single-threaded {p1} passes in {el1:.1f} s",
            "cpu_model": cpu_model(), "usable_cores": usable_cores(1 << 30),
            "single_thread": {"value": round(rate(p1, el1), 4), "unit": unit, "passes": p1,
                              "phases_s": {k: round(v, 3) for k, v in ph1.items()}},
            "all_cores": {"value": round(rate(pn, eln), 4), "unit": unit, "passes": pn, "cores": cores,
                          "phases_s": {k: round(v, 3) for k, v in phn.items()}},
            "offline_scale_and_codes_s": round(pack_s, 3)}


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
    kernel = dominant_kernel_name(spec, args)

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


# The two counter passes of --summarize-sq (eight SQ counters each: one pass holds at most eight).
SQ_PASSES = (["SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_WAIT_INST_LDS",
              "SQ_ACTIVE_INST_ANY", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_LDS_BANK_CONFLICT"],
             ["SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS", "SQ_ACTIVE_INST_VMEM", "SQ_ACTIVE_INST_MISC",
              "SQ_INSTS_LDS", "SQ_LDS_ADDR_CONFLICT", "SQ_INST_LEVEL_LDS", "SQ_WAVES"])


def summarize_sq(args):
    """Per-shape wave-time breakdown of k_gemm on the prefill workload from two rocprofv3 --pmc passes
    (SQ_PASSES), summed over every dispatch of each shape: issuing, VALU share of issue, waiting at
    s_waitcnt, dependency stalls, LDS bank conflicts per LDS instruction. A dispatch's shape is told
    by its grid, sized as the GEMM launcher sizes it (the step's route: workspace and split plan)."""
    d1, d2, out_md = args.summarize_sq
    spec = workload_spec(args.workload, args.m)
    if not spec["prefill"]:
        raise SystemExit("--summarize-sq is for the prefill workload")
    import bit_ternary_weight_absmean_amd as bt

    M = spec["M"]
    label = {}
    for name, N, K in spec["shapes"]:
        tiles = -(-M // 64) * -(-N // 256)
        full, splits = bt.gemm_split_plan(M, N, K)
        full = tiles if splits == 1 else full
        wgs = 8 * (-(-full // 8) + -(-(tiles - full) // 8) * splits)
        split = "" if splits == 1 else (f", {full} whole + {tiles - full} split in {splits}" if full
                                        else f", every tile split in {splits}")
        label[wgs * 256] = f"{name} {N}x{K} ({tiles} tiles{split})"
    sums = collections.defaultdict(lambda: collections.defaultdict(float))
    for d, counters in zip((d1, d2), SQ_PASSES):
        for c in counters:
            for r in _pmc_rows(d, c):
                if "k_gemm<" in r["Kernel_Name"]:
                    sums[int(r["Grid_Size"])][c] += float(r["Counter_Value"])
    cmd = ("rocprofv3 --pmc {} --output-format csv -d gpurun_out/{} -o run -- python3 bench.py --workload "
           f"2b_prefill --m {M} --eager --steps 1 --warmup 1 --no-cpu-baseline --no-ceilings")
    lines = [f"# k_gemm wave-time breakdown on the 2B prefill workload (M={M}), per shape", "",
             "Commands (run from the repository root, one pass per counter set), then "
             f"`python3 bench.py --workload 2b_prefill --m {M} --summarize-sq gpurun_out/sq1 gpurun_out/sq2 <this file>`:",
             "", "    " + cmd.format(" ".join(SQ_PASSES[0]), "sq1"), "    " + cmd.format(" ".join(SQ_PASSES[1]), "sq2"),
             "", f"k_gemm source sha256 (comments and blank lines out): `{source_hash('k_gemm')}`.", "",
             "Sums over every dispatch of each shape in the run. Per-wave cycles are SQ_WAVE_CYCLES / SQ_WAVES (the "
             "counter's own units); the shares are of SQ_WAVE_CYCLES.", "",
             "| shape | waves | wave-cycles per wave | issuing (ACTIVE_INST_ANY) | of which VALU | at s_waitcnt "
             "(WAIT_ANY) | dependency / issue stalls (WAIT_INST_ANY) | LDS bank conflicts per LDS instruction |",
             "|---|---|---|---|---|---|---|---|"]
    for grid, c in sorted(sums.items(), key=lambda kv: kv[1]["SQ_WAVES"]):
        wc = c["SQ_WAVE_CYCLES"] or 1.0
        lines.append("| {} | {:.0f} | {:.0f} | {:.0%} | {:.0%} | {:.0%} | {:.0%} | {:.2f} |".format(
            label.get(grid, f"grid {grid}"), c["SQ_WAVES"], wc / max(c["SQ_WAVES"], 1.0),
            c["SQ_ACTIVE_INST_ANY"] / wc, c["SQ_ACTIVE_INST_VALU"] / max(c["SQ_ACTIVE_INST_ANY"], 1.0),
            c["SQ_WAIT_ANY"] / wc, c["SQ_WAIT_INST_ANY"] / wc,
            c["SQ_LDS_BANK_CONFLICT"] / max(c["SQ_INSTS_LDS"], 1.0)))
    with open(out_md, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_trace(args):
    """Per-kernel summary of a rocprofv3 --kernel-trace --stats run of this workload: for every
    kernel of this library, launches, mean and median duration (end - start of each dispatch)
    and the mean interval from one dispatch's start to the next one's when they follow each
    other inside a replayed graph (next start within 50 us). The interval is the per-launch
    time the benchmark's HIP events measure (graph time over launches): short dispatches of a
    graph overlap their completion with the next one's start, so their durations can sum to
    more than the graph's time."""
    import statistics

    # TRACE_DIR may list several runs of the same command, comma-separated: the tables cover
    # them all, and the dominant kernel's figure is the median of the runs' means (the tracer's
    # spacing of dispatches, and so a short kernel's traced duration, varies from run to run)
    trace_dirs, out_md = args.summarize_trace[0].split(","), args.summarize_trace[1]

    def load(trace_dir):
        files = glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True)
        if not files:
            raise SystemExit(f"no kernel_trace.csv under {trace_dir}")
        rows = []
        for f in files:
            with open(f) as fh:
                rows += list(csv.DictReader(fh))
        rows.sort(key=lambda r: int(r["Start_Timestamp"]))
        per = collections.OrderedDict()
        for i, r in enumerate(rows):
            name = r["Kernel_Name"]
            if not any(k in name for k in ("k_linear_decode", "k_gemv", "k_gemm", "k_quant_act", "k_read", "k_empty",
                                           "k_store_one", "k_mfma_loop", "k_pack", "k_gamma", "k_row_abs_sum")):
                continue
            start, end = int(r["Start_Timestamp"]), int(r["End_Timestamp"])
            key = (name, r.get("Grid_Size", r.get("Grid_Size_X", "")),
                   r.get("Workgroup_Size", r.get("Workgroup_Size_X", "")))
            e = per.setdefault(key, {"dur": [], "gap": []})
            e["dur"].append((end - start) / 1e3)
            if i + 1 < len(rows):
                nxt = int(rows[i + 1]["Start_Timestamp"])
                if 0 <= nxt - start <= 50_000:
                    e["gap"].append((nxt - start) / 1e3)
        return per

    runs = [load(d) for d in trace_dirs]
    per = collections.OrderedDict()
    for pr in runs:
        for key, e in pr.items():
            m = per.setdefault(key, {"dur": [], "gap": []})
            m["dur"] += e["dur"]
            m["gap"] += e["gap"]
    trace_dir = trace_dirs[0]
    lines = [f"# Kernel trace: {args.workload} workload" + (f" (M={args.m})" if args.m else ""), "",
             "Command (run from the repository root):", "", f"    {args.command}", "",
             "Per kernel instance and launch shape: dispatch durations (end - start) and the interval from a",
             "dispatch's start to the next dispatch's start inside a replayed graph (next start within 50 us;",
             "the per-launch time that the benchmark's HIP events measure as graph time over launches).", "",
             "| kernel | grid | WG | launches | mean us | median us | intervals | mean interval us | "
             "median interval us |", "|---|---|---|---|---|---|---|---|---|"]
    for (name, grid, wg), e in per.items():
        d, gp = e["dur"], e["gap"]
        lines.append(f"| `{name}` | {grid} | {wg} | {len(d)} | {statistics.mean(d):.3f} | {statistics.median(d):.3f} "
                     f"| {len(gp)} | {statistics.mean(gp) if gp else float('nan'):.3f} | "
                     f"{statistics.median(gp) if gp else float('nan'):.3f} |")
    def is_kernel(name, kname):  # k_gemm, not k_gemm_ks; k_gemv_direct and k_gemv_direct_db
        return re.search(rf"\b{kname}(_db)?[<(]", name) is not None

    # every product kernel of the workload together
    for kname in ("k_linear_decode", "k_gemv_staged", "k_gemv_blocked", "k_gemv_direct", "k_gemv_lut", "k_gemv_bits",
                  "k_gemm", "k_gemm_ks"):
        d = [x for (n, _, _), e in per.items() if is_kernel(n, kname) for x in e["dur"]]
        gp = [x for (n, _, _), e in per.items() if is_kernel(n, kname) for x in e["gap"]]
        if d:
            lines += ["", f"All `{kname}` dispatches: {len(d)}, mean duration {statistics.mean(d):.3f} us, "
                          f"mean interval {statistics.mean(gp) if gp else float('nan'):.3f} us over {len(gp)} "
                          "back-to-back pairs."]
    stats = glob.glob(os.path.join(trace_dir, "**", "*kernel_stats.csv"), recursive=True)
    if stats:
        lines += ["", "rocprofv3 `--stats` (kernel_stats.csv), this library's kernels:", "",
                  "| kernel | calls | avg ns | min ns | max ns |", "|---|---|---|---|---|"]
        with open(stats[0]) as fh:
            for r in csv.DictReader(fh):
                if any(k in r["Name"] for k in ("k_linear_decode", "k_gemv", "k_gemm", "k_quant_act", "k_read",
                                                "k_empty", "k_store_one", "k_mfma_loop")):
                    lines.append(f"| `{r['Name']}` | {r['Calls']} | {float(r['AverageNs']):.0f} | "
                                 f"{float(r['MinNs']):.0f} | {float(r['MaxNs']):.0f} |")
    # the workload's dominant kernel, for the benchmark line (read back while the sources match)
    spec = workload_spec(args.workload, args.m)
    kname = dominant_kernel_name(spec, args)
    d = [x for (n, _, _), e in per.items() if is_kernel(n, kname) for x in e["dur"]]
    gp = [x for (n, _, _), e in per.items() if is_kernel(n, kname) for x in e["gap"]]
    # one figure per launch only where every matrix of the step runs that kernel
    single = all(re.search(rf"\b{kname}<", p) for p in step_plans(spec, getattr(args, "split", False)))
    if d and not single:
        kernels = dict.fromkeys(k for p in step_plans(spec) for k in re.findall(r"k_\w+", p) if "quant" not in k)
        lines += ["", f"The step runs more than one product kernel ({', '.join(kernels)}): no single",
                  "per-launch figure is recorded for it."]
    if d and single:
        M = spec["M"]
        alg = [linear_bytes(M, N, K) if kname == "k_linear_decode" else gemv_bytes(M, N, K)
               for _, N, K in spec["shapes"]]
        ops = [2 * M * N * K for _, N, K in spec["shapes"]]
        run_means = [statistics.mean([x for (n, _, _), e in pr.items() if is_kernel(n, kname) for x in e["dur"]])
                     for pr in runs]
        rec = {"kernel": kname, "workload": spec["desc"], "M": M, "source_sha256": source_hash(kname),
               "dispatches": len(d), "mean_duration_us": round(statistics.median(run_means), 3),
               "run_mean_duration_us": [round(x, 3) for x in run_means],
               "mean_interval_us": round(statistics.mean(gp), 3) if gp else None,
               "algorithmic_bytes_per_launch": round(sum(alg) / len(alg)),
               "ops_per_launch": round(sum(ops) / len(ops)), "command": args.command}
        with open(os.path.splitext(out_md)[0] + ".json", "w") as fh:
            json.dump(rec, fh, indent=1)
            fh.write("\n")
        lines += ["", f"Dominant kernel of the workload: `{kname}`, {len(d)} dispatches over {len(runs)} run(s), mean "
                      f"duration per run {', '.join(f'{x:.3f}' for x in run_means)} us, median "
                      f"{rec['mean_duration_us']} us; algorithmic bytes per launch {rec['algorithmic_bytes_per_launch']} "
                      f"-> {rec['algorithmic_bytes_per_launch'] / rec['mean_duration_us'] / 1e3:.1f} GB/s, "
                      f"{rec['ops_per_launch'] / rec['mean_duration_us'] / 1e6:.1f} TOP/s at the traced mean.",
                  "",
                  "How this relates to the benchmark line: `roofline.achieved` divides the algorithmic bytes (or",
                  "ops) per launch by the per-launch time of the step's HIP graph measured with HIP events",
                  "(`detail.launch_interval_us`). Under the tracer the graph's dispatches are spaced several",
                  "microseconds apart (see the interval columns; the empty kernel shows the same spacing), so each",
                  "dispatch above ran alone from a cold start, and its mean duration is the conservative figure the",
                  "line reports as `detail.traced` (read from the JSON next to this file while the kernel's",
                  "sources are unchanged; with several runs, the median of their means)."]
    with open(out_md, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def dominant_kernel_name(spec, args):
    """The product kernel the workload's step runs (as run_gpu picks it)."""
    import bit_ternary_weight_absmean_amd as bt

    M = spec["M"]
    if not getattr(args, "split", False) and all(bt.linear_workspace_bytes(M, N, K) == 0 for _, N, K in spec["shapes"]):
        return "k_linear_decode"
    if spec["prefill"] or M > bt.GEMV_MAX_M:
        return "k_gemm"
    return "k_gemv_staged"


def traced_for(spec, kernel):
    """The committed trace summary of the workload's dominant kernel, while its sources match."""
    if ROW_SCALES:
        return None
    path = os.path.join(ROOT, "profiles", f"trace_{kernel}_{spec['name']}_m{spec['M']}.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("source_sha256") != source_hash(kernel):
        return None
    return rec


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
def prefill_detail(args, g, spec):
    """The metric's second half: the 2B prefill GEMM step at M = 2048 (quantizer + GEMM per
    matrix) and the GEMM launches alone against the int8 MFMA roofline."""
    gemm_us = g["ms_prod"] * 1e3 / g["n_prod"]
    ops_per_launch = g["step_ops"] / g["n_prod"]
    ach = ops_per_launch / (gemm_us * 1e-6) / 1e12
    return {"workload": spec["desc"], "M": spec["M"], "shapes": [f"{n} {N}x{K}" for n, N, K in spec["shapes"]],
            "ms_per_step": round(g["ms_step"], 5), "step_TOPS": round(g["step_ops"] / (g["ms_step"] * 1e-3) / 1e12, 1),
            "kernel": g["kernel"], "kernel_us_per_launch": round(gemm_us, 3),
            "kernel_us_per_shape": {n: round(u, 3) for (n, _, _), u in zip(spec["shapes"], g["shape_us"])},
            "roofline": {"bound": "mfma", "achieved": round(ach, 1), "peak": INT8_PEAK_TOPS, "unit": "TOP/s",
                         "frac": round(ach / INT8_PEAK_TOPS, 4), "traffic": traffic_for(spec, "k_gemm")},
            "mfma_util_percent_counters": mfma_util_for(spec, "k_gemm"),
            "traced": traced_summary(spec, "k_gemm")}


# The other configurations the default run measures besides the metric's two halves (2B decode
# at one token, 2B prefill at 2048): each step timed as the main line's, reported compactly.
EXTRA_WORKLOADS = [("2b_decode", 4), ("7b_decode", 1), ("7b_decode", 4), ("7b_decode", 8), ("2b_prefill", 256),
                   ("100b_decode", 1), ("100b_decode", 16)]


def workload_summary(args, name, M):
    """One configuration's step: time, rate against its roofline (HBM for decode, int8 MFMA for
    prefill), the per-launch interval of its product kernels and each shape's time in the step."""
    spec = workload_spec(name, M)
    if ROW_SCALES:
        spec["desc"] += ", row-group weight scales (one per Q, K, V and gate, up block)"
    g = run_gpu(args, spec)
    prod_us = g["ms_prod"] * 1e3 / g["n_prod"]
    out = {"workload": spec["desc"], "M": M, "layers": spec["layers"], "ms_per_step": round(g["ms_step"], 5),
           "kernel": g["kernel"], "launch_interval_us": round(prod_us, 3),
           "kernel_us_per_shape": {n: round(u, 3) for (n, _, _), u in zip(spec["shapes"], g["shape_us"])}}
    if spec["prefill"]:
        ach = g["step_ops"] / g["n_prod"] / (prod_us * 1e-6) / 1e12
        out.update(step_TOPS=round(g["step_ops"] / (g["ms_step"] * 1e-3) / 1e12, 1), product_TOPS=round(ach, 1),
                   frac_of_int8_peak=round(ach / INT8_PEAK_TOPS, 4))
    else:
        gbs = g["step_bytes"] / (g["ms_step"] * 1e-3) / 1e9
        out.update(step_GBs=round(gbs, 1), frac_of_hbm_peak=round(gbs / HBM_PEAK_GBS, 4))
    g.pop("packed")
    return out


def traced_summary(spec, kernel):
    tr = traced_for(spec, kernel)
    if tr is None:
        return None
    t_ach = (tr["ops_per_launch"] / (tr["mean_duration_us"] * 1e-6) / 1e12 if spec["prefill"]
             else tr["algorithmic_bytes_per_launch"] / (tr["mean_duration_us"] * 1e-6) / 1e9)
    return {"source": f"profiles/trace_{kernel}_{spec['name']}_m{spec['M']}.json",
            "mean_duration_us": tr["mean_duration_us"], "achieved": round(t_ach, 1),
            "frac": round(t_ach / (INT8_PEAK_TOPS if spec["prefill"] else HBM_PEAK_GBS), 4)}


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
    if args.summarize_sq:
        summarize_sq(args)
        return 0
    if args.summarize_trace:
        summarize_trace(args)
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
        roof = {"bound": "mfma", "achieved": round(ach, 1), "peak": INT8_PEAK_TOPS, "unit": "TOP/s",
                "frac": round(ach / INT8_PEAK_TOPS, 4), "traffic": traffic}
    else:
        value = g["step_bytes"] / (g["ms_step"] * 1e-3) / 1e9
        unit = "GB/s"
        ach = bytes_per_launch / (prod_us * 1e-6) / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": traffic}
    ceil = None
    if not args.no_ceilings:
        ceil = run_ceilings(args, spec, g)
    prefill = None
    if args.workload == "2b_decode" and not args.no_prefill and not args.split:
        # the metric's prefill half, in the same run: 2B prefill at 2048 tokens
        pspec = workload_spec("2b_prefill", 2048)
        if ROW_SCALES:
            pspec["desc"] += ", row-group weight scales (one per Q, K, V and gate, up block)"
        g.pop("packed")
        gp = run_gpu(args, pspec)
        prefill = prefill_detail(args, gp, pspec)
        if ceil is not None:
            prefill["roofline"]["achievable"] = ceil["mfma_int8_TOPS"]
            prefill["roofline"]["frac_of_achievable"] = round(prefill["roofline"]["achieved"] /
                                                              ceil["mfma_int8_TOPS"], 4)
        del gp
    elif spec["prefill"] and ceil is not None:
        roof["achievable"] = ceil["mfma_int8_TOPS"]
        roof["frac_of_achievable"] = round(ach / ceil["mfma_int8_TOPS"], 4)
    workloads = None
    if args.workload == "2b_decode" and M == 1 and not args.no_workloads and not args.split:
        g.pop("packed", None)
        workloads = [workload_summary(args, n, m) for n, m in EXTRA_WORKLOADS]
    cpu = None if args.no_cpu_baseline else run_cpu_baseline(args, spec)
    detail = {"dominant_kernel": g["kernel"],
              "launch_interval_us": round(prod_us, 3),
              "launch_interval_note": "product launches of one step replayed as a HIP graph, timed with HIP "
                                      "events on their stream, divided by the launches: the per-launch time "
                                      "roofline.achieved uses",
              "kernel_us_per_shape": {n: round(u, 3) for (n, _, _), u in zip(spec["shapes"], g["shape_us"])},
              "algorithmic_bytes_per_launch": round(bytes_per_launch),
              "ops_per_launch": round(ops_per_launch),
              "step_hbm_frac": None if spec["prefill"] else round(value / HBM_PEAK_GBS, 4),
              "step_TOPS": round(g["step_ops"] / (g["ms_step"] * 1e-3) / 1e12, 3),
              "weights_per_s": round(sum(N * K for _, N, K in spec["shapes"]) * spec["layers"] /
                                     (g["ms_step"] * 1e-3), 1),
              "setup_s": round(g["setup_s"], 1),
              "mfma_util_percent_counters": mfma_util_for(spec, g["kernel"]) if spec["prefill"] else None}
    # the same launches under rocprofv3 --kernel-trace (committed summary): the tracer spaces the
    # dispatches apart, so each runs from a cold start; its mean duration is the conservative figure
    detail["traced"] = traced_summary(spec, g["kernel"])
    if ceil is not None:
        detail["launch_floor_us"] = ceil["launch_floor_us"]
        detail["ceilings"] = ceil
        if not spec["prefill"]:
            detail["step_frac_of_read_ceiling"] = ceil["step_frac_of_read_step"]
    if prefill is not None:
        detail["prefill"] = prefill
    if workloads is not None:
        detail["workloads"] = workloads
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
                            else "per matrix: bt_ternary_linear (the fused decode kernel where it takes the "
                                 "shape, else bt_quant_act + bt_ternary_gemv)" if g["fused_any"]
                            else ("per matrix: bt_quant_act + " if args.split else
                                  "per matrix: bt_ternary_linear = bt_quant_act + ") +
                            ("bt_ternary_gemm_ws" if "k_gemm" in g["kernel"] else "bt_ternary_gemv"))},
        "roofline": roof,
        "cpu_baseline": cpu,
        "detail": detail,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
