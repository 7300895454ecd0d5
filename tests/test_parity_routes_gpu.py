"""GPU parity on the launches the benchmark times.

Every workload ``bench.py`` measures (2B, 7B and 100B-class decode, 2B-class prefill), at
every token count it is measured at, through each route it can time:

* ``linear``: bt_ternary_linear (one fused launch at decode sizes; quantizer + staged or
  direct GEMV, or quantizer + split-K GEMM, past them) -- the default step;
* ``split``: bt_quant_act, then bt_ternary_gemv (BT_GEMV_AUTO) or bt_ternary_gemm_ws
  (``--split``);
* ``rows``: bt_ternary_linear_rs on weights packed with one scale per Q, K, V and gate, up
  block (``--row-scales``);
* ``split_rows``: bt_quant_act, then bt_ternary_gemv_rs or bt_ternary_gemm_rs on those
  weights (``--split --row-scales``).

Inputs are the workloads' own seeded activations and seeded weights of their shapes.
Matrices of at most 22016 rows are compared on every output row; larger ones on two rows
of every 64-row block. Prefill outputs are compared on token rows sampled in every
64-token tile row. Bar: acc bit-exact; Y within |dY| <= 1e-5 |Y| + 1e-6. The oracle result
of the largest token count serves the smaller ones: activation rows are per-token
independent and the smaller draws are prefixes of the larger.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import bit_ternary_weight_absmean_amd as bt
from bit_ternary_weight_absmean_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

# workload -> (seed config, layer shapes, token counts): the workloads bench.py times
# (tests/test_plan_coverage.py checks every kernel instance they launch against these).
ROUTE_WORKLOADS = {
    "2b_decode": (synth.CFG_2B_DECODE, synth.SHAPES_2B, (1, 4)),
    "7b_decode": (synth.CFG_7B_DECODE, synth.SHAPES_7B, (1, 2, 4, 8)),
    "100b_decode": (synth.CFG_100B_DECODE, synth.SHAPES_100B, (1, 2, 4, 16)),
    "2b_prefill": (synth.CFG_2B_PREFILL, synth.SHAPES_2B, (256, 2048)),
}
ROUTES = ("linear", "split", "rows", "split_rows")
FULL_ROWS_MAX = 22016


def route_cases():
    """(workload, matrix index, route) of every parity case below, in a stable order."""
    return [(w, j, r) for w, (_, shapes, _) in ROUTE_WORKLOADS.items() for j in range(len(shapes)) for r in ROUTES]


def note(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def tol_ok(y, ref):
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    return bool(np.all(np.abs(y - ref) <= 1e-5 * np.abs(ref) + 1e-6))


def compare_rows(N):
    """Output rows compared: all of them up to FULL_ROWS_MAX, else two per 64-row block
    (offsets vary from block to block) and the last row."""
    if N <= FULL_ROWS_MAX:
        return np.arange(N)
    blocks = np.arange(0, N, 64)
    a = blocks + (blocks // 64 * 7) % 64
    b = blocks + 63 - (blocks // 64 * 13) % 32
    rows = np.unique(np.concatenate([a, b, [N - 1]]))
    return rows[rows < N]


_WEIGHTS = {}


def weights(workload, j, rows_mode):
    """(packed weights on the device, compared row indices, codes of those rows, their
    scale(s)) for matrix j of the workload, cached for the module."""
    key = (workload, j, rows_mode)
    if key in _WEIGHTS:
        return _WEIGHTS[key]
    cfg, shapes, _ = ROUTE_WORKLOADS[workload]
    name, N, K = shapes[j]
    W = synth.layer_weight(cfg, 0, j, N, K)
    rows = compare_rows(N)
    if rows_mode:
        groups = synth.row_groups(cfg, name, N)
        rs = oracle.absmean_rows(W, list(groups))
        T = oracle.ternarize_rows(W[rows], rs[rows])
        pw = bt.pack_weights_rows(torch.from_numpy(W).to(DEV), list(groups))
        scale = rs[rows]
        assert np.array_equal(pw.scale.cpu().numpy().view(np.uint32), rs.view(np.uint32))
    else:
        g = oracle.absmean(W)
        T = oracle.ternarize(W[rows], g)
        pw = bt.pack_weights(torch.from_numpy(W).to(DEV))
        scale = g
        assert pw.scale.cpu().numpy().view(np.uint32)[0] == np.float32(g).view(np.uint32)
    del W
    _WEIGHTS[key] = (pw, rows, T, scale)
    return _WEIGHTS[key]


_REFS = {}


def reference(workload, j, rows_mode, M, toks, Xmax, T, scale):
    """Oracle acc and Y on the compared tokens and rows (shared by the routes of one packing)."""
    key = (workload, j, rows_mode, M)
    if key not in _REFS:
        Q, s, _ = oracle.quant_act(Xmax[toks])
        acc_ref = oracle.ternary_matmul(T, Q)
        Y_ref = (oracle.scale_epilogue_rows(acc_ref, scale, s) if rows_mode
                 else oracle.scale_epilogue(acc_ref, scale, s))
        _REFS[key] = (acc_ref, Y_ref)
    return _REFS[key]


def token_rows(M, prefill):
    if not prefill:
        return np.arange(M)
    return np.unique(np.concatenate([np.arange(0, M, 61), [M - 1]]))


def run_route(route, pw, X, M, N, K, prefill):
    Xd = torch.from_numpy(X).to(DEV)
    if route in ("linear", "rows"):
        ws_bytes = bt.linear_workspace_bytes(M, N, K)
        # a workspace full of garbage: the call initializes everything it reads
        ws = torch.full((ws_bytes,), 0xFF, dtype=torch.uint8, device=DEV) if ws_bytes else None
        Y, acc = bt.linear(Xd, pw, want_acc=True, workspace=ws)
    else:
        q = bt.quant_act(Xd)
        if prefill or M > bt.GEMV_MAX_M:
            Y, acc = bt.ternary_gemm(pw, q, want_acc=True, workspace=bt.gemm_workspace(M, N, K, DEV))
        else:
            Y, acc = bt.ternary_gemv(pw, q, want_acc=True, algo=bt.GEMV_AUTO)
    torch.cuda.synchronize()
    return Y.cpu().numpy(), acc.cpu().numpy()


@pytest.mark.parametrize("workload,j,route", route_cases())
def test_bench_route(workload, j, route):
    cfg, shapes, Ms = ROUTE_WORKLOADS[workload]
    name, N, K = shapes[j]
    prefill = workload.endswith("prefill")
    rows_mode = route in ("rows", "split_rows")
    pw, rows, T, scale = weights(workload, j, rows_mode)
    Xmax = synth.layer_activation(cfg, j, max(Ms), K)
    for M in Ms:
        note(f"{workload} {name} {N}x{K} M={M} route={route} plan={bench_plan(route, M, N, K, prefill)}")
        toks = token_rows(M, prefill)
        acc_ref, Y_ref = reference(workload, j, rows_mode, M, toks, Xmax, T, scale)
        Y, acc = run_route(route, pw, np.ascontiguousarray(Xmax[:M]), M, N, K, prefill)
        assert acc.shape == (M, N)
        got = acc[np.ix_(toks, rows)]
        bad = np.argwhere(got != acc_ref)
        assert bad.size == 0, f"{len(bad)} acc mismatches at M={M}, first (token, row) {bad[:5].tolist()}"
        assert tol_ok(Y[np.ix_(toks, rows)], Y_ref), f"Y outside tolerance at M={M}"


def bench_plan(route, M, N, K, prefill):
    """The kernel instances of this case (bt_kernel_plan), printed with the case name."""
    rows = route in ("rows", "split_rows")
    if route in ("linear", "rows"):
        return bt.kernel_plan(bt.CALL_LINEAR, M, N, K, row_scales=rows)
    if prefill or M > bt.GEMV_MAX_M:
        return bt.kernel_plan(bt.CALL_QUANT, M, N, K) + " + " + bt.kernel_plan(bt.CALL_GEMM_WS, M, N, K,
                                                                               row_scales=rows)
    return bt.kernel_plan(bt.CALL_QUANT, M, N, K) + " + " + bt.kernel_plan(bt.CALL_GEMV, M, N, K, bt.GEMV_AUTO,
                                                                           row_scales=rows)
