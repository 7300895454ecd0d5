"""GPU parity on seeded random shapes: the product entry points against the oracle.

The shapes are drawn once from a fixed seed, so every run checks the same set: tokens M
from 1 to 600, rows N from 1 to 4000, inputs K from 1 to 9000, each log-uniform so that the
small and ragged ends are drawn as often as the large ones, with M * N * K at most 1e9 so
that the oracle finishes a case in well under a second. Every shape runs:

* bt_ternary_linear, on whatever route the library picks for it (the fused decode kernel;
  quantizer + the staged, blocked or direct GEMV; quantizer + the small-M GEMM form or the
  64 x 256 GEMM, whole or split), and bt_ternary_linear_static on every fourth shape;
* bt_ternary_gemm with and without its workspace;
* for M <= 16, bt_ternary_gemv with every kernel choice that takes the shape;
* on every third shape, the same weights packed with row-group scales through
  bt_ternary_linear_rs.

Bar: acc bit-exact and Y within |dY| <= 1e-5 |Y| + 1e-6 on every output.
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


def _shapes(n=60, seed=20261203, max_ops=1e9):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        M, N, K = (int(np.exp(rng.uniform(0.0, np.log(hi + 1)))) for hi in (600, 4000, 9000))
        M, N, K = max(M, 1), max(N, 1), max(K, 1)
        if M * N * K <= max_ops:
            out.append((M, N, K))
    return out


SHAPES = _shapes()


def note(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def tol_ok(y, ref):
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    return bool(np.all(np.abs(y - ref) <= 1e-5 * np.abs(ref) + 1e-6))


def check(name, Y, acc, ref):
    torch.cuda.synchronize()
    a = acc.cpu().numpy()
    bad = np.argwhere(a != ref["acc"])
    assert bad.size == 0, f"{name}: {len(bad)} acc mismatches, first at {bad[:5].tolist()}"
    assert tol_ok(Y.cpu().numpy(), ref["Y"]), f"{name}: Y outside tolerance"


def gemv_algos(M, K):
    """The kernel choices of bt_ternary_gemv_algo that take M tokens of K inputs."""
    algos = [bt.GEMV_AUTO, bt.GEMV_STAGED, bt.GEMV_MFMA]
    if M <= 4:
        algos.append(bt.GEMV_DOT4)
    if M == 1 and K <= 6912:
        algos.append(bt.GEMV_LUT)
    return algos


@pytest.mark.parametrize("case", range(len(SHAPES)))
def test_random_shape(case):
    M, N, K = SHAPES[case]
    plan = bt.kernel_plan(bt.CALL_LINEAR, M, N, K)
    note(f"random case {case}: M={M} N={N} K={K} linear plan={plan}")
    W = synth.gaussian((N, K), 31000 + case, 0.02)
    X = synth.gaussian((M, K), 32000 + case)
    ref = oracle.linear(W, X)
    pw = bt.pack_weights(torch.from_numpy(W).to(DEV))
    Xd = torch.from_numpy(X).to(DEV)

    Y, acc = bt.linear(Xd, pw, want_acc=True)
    check("linear", Y, acc, ref)
    if case % 4 == 0:
        Y, acc = bt.linear_static(Xd, pw, want_acc=True)
        check("linear_static", Y, acc, ref)

    q = bt.quant_act(Xd)
    Y, acc = bt.ternary_gemm(pw, q, want_acc=True)
    check("gemm", Y, acc, ref)
    ws = bt.gemm_workspace(M, N, K, DEV)
    if ws is not None:
        Y, acc = bt.ternary_gemm(pw, q, want_acc=True, workspace=ws)
        check("gemm_ws", Y, acc, ref)
    if M <= bt.GEMV_MAX_M:
        for algo in gemv_algos(M, K):
            Y, acc = bt.ternary_gemv(pw, q, want_acc=True, algo=algo)
            check(f"gemv algo {algo}", Y, acc, ref)

    if case % 3 == 0 and N >= 2:
        groups = [N // 2, N - N // 2] if N < 8 else [N // 4, N // 2, N - N // 4 - N // 2]
        Wg = W * np.repeat(np.float32([1.0, 8.0, 0.25])[:len(groups)], groups)[:, None]
        ref_rows = oracle.linear_rows(Wg, X, groups)
        pwr = bt.pack_weights_rows(torch.from_numpy(Wg).to(DEV), groups)
        Y, acc = bt.linear(Xd, pwr, want_acc=True)
        check("linear_rs", Y, acc, ref_rows)
