"""GPU parity of the row-group weight scales against the CPU oracle.

bt_pack_weights_rows (row scales and codes bit-exact), and the products and the linear
layer taking those scales (acc bit-exact, Y within |dY| <= 1e-5 |Y| + 1e-6), on every
route: the fused decode kernel, the direct and dot4 GEMVs and the prefill GEMM with and
without its split-K workspace.
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


def note(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def tol_ok(y, ref):
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    return bool(np.all(np.abs(y - ref) <= 1e-5 * np.abs(ref) + 1e-6))


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def grouped(N, K, groups, seed):
    """W ~ 0.02 N(0,1) with each group at its own magnitude, so that a scale taken over the
    wrong rows changes the codes of whole groups."""
    W = synth.gaussian((N, K), seed, 0.02)
    if groups is None:
        W *= np.exp2(np.arange(N) % 7 - 3).astype(np.float32)[:, None]
        return W
    n0 = 0
    for i, rows in enumerate(groups):
        W[n0:n0 + rows] *= np.float32([1.0, 12.0, 0.125, 3.0][i % 4])
        n0 += rows
    return W


# (N, K, groups): explicit groups, one group per row (None), one group, and the 2B
# fused projections (QKV = 2560 + 640 + 640 rows, gate+up = 6912 + 6912).
PACK_CASES = [(768, 300, [640, 64, 64]), (200, 129, None), (130, 517, [130]), (96, 64, [1, 94, 1]),
              (70, 8, [10, 20, 30, 10]), (3840, 2560, [2560, 640, 640]), (13824, 2560, [6912, 6912])]


@pytest.mark.parametrize("N,K,groups", PACK_CASES)
def test_pack_rows(N, K, groups):
    note(f"pack_rows N={N} K={K} groups={groups}")
    W = grouped(N, K, groups, 8100 + N + K)
    pw = bt.pack_weights_rows(to_dev(W), groups)
    T = bt.unpack_weights(pw)
    torch.cuda.synchronize()
    rs_ref = oracle.absmean_rows(W, groups)
    np.testing.assert_array_equal(pw.scale.cpu().numpy()[:N].view(np.uint32), rs_ref.view(np.uint32))
    np.testing.assert_array_equal(T.cpu().numpy(), oracle.ternarize_rows(W, rs_ref))


def test_pack_rows_empty_k():
    note("pack_rows K=0")
    W = torch.zeros((5, 0), dtype=torch.float32, device=DEV)
    pw = bt.pack_weights_rows(W, [2, 3])
    torch.cuda.synchronize()
    assert np.all(pw.scale.cpu().numpy()[:5] == 0.0)


# (M, N, K, groups) on each route of bt_ternary_linear_rs: fused (M <= 4), quantizer +
# direct GEMV (M <= 16), quantizer + GEMM (M > 16: here the small-M form k_gemm_ks, whose
# few tiles split their k-steps inside the workgroup).
LINEAR_CASES = [(1, 768, 300, [640, 64, 64]), (3, 200, 1000, None), (4, 130, 517, [130]),
                (1, 3840, 2560, [2560, 640, 640]), (2, 9000, 1000, [4500, 4500]),
                (8, 768, 700, [640, 64, 64]), (16, 600, 2560, None),
                (40, 768, 700, [640, 64, 64]), (100, 2500, 6900, [1000, 1500]), (300, 257, 1000, None),
                (520, 2100, 700, [1000, 1100])]


@pytest.mark.parametrize("M,N,K,groups", LINEAR_CASES)
def test_linear_rows(M, N, K, groups):
    note(f"linear_rs M={M} N={N} K={K} groups={groups}")
    W = grouped(N, K, groups, 8300 + N + K)
    X = synth.gaussian((M, K), 8400 + M + K)
    ref = oracle.linear_rows(W, X, groups)
    pw = bt.pack_weights_rows(to_dev(W), groups)
    Y, acc = bt.linear(to_dev(X), pw, want_acc=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(acc.cpu().numpy(), ref["acc"])
    assert tol_ok(Y.cpu().numpy(), ref["Y"])


@pytest.mark.parametrize("M,algo", [(1, bt.GEMV_DOT4), (3, bt.GEMV_DOT4), (1, bt.GEMV_MFMA), (5, bt.GEMV_MFMA),
                                    (16, bt.GEMV_MFMA)])
def test_gemv_rows(M, algo):
    N, K, groups = 768, 700, [640, 64, 64]
    note(f"gemv_rs M={M} algo={algo}")
    W = grouped(N, K, groups, 8500 + M)
    X = synth.gaussian((M, K), 8600 + M)
    ref = oracle.linear_rows(W, X, groups)
    pw = bt.pack_weights_rows(to_dev(W), groups)
    Y, acc = bt.ternary_gemv(pw, bt.quant_act(to_dev(X)), want_acc=True, algo=algo)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(acc.cpu().numpy(), ref["acc"])
    assert tol_ok(Y.cpu().numpy(), ref["Y"])


def test_gemm_rows_split_and_plain():
    M, N, K, groups = 700, 3000, 4000, [2000, 500, 500]
    note(f"gemm_rs M={M} N={N} K={K}")
    W = grouped(N, K, groups, 8700)
    X = synth.gaussian((M, K), 8701)
    rows = np.concatenate([np.arange(3, M, 29), [M - 1]])  # token rows in every 64-token tile row
    ref = oracle.linear_rows(W, X[rows], groups)
    pw = bt.pack_weights_rows(to_dev(W), groups)
    q = bt.quant_act(to_dev(X))
    ws = bt.gemm_workspace(M, N, K, DEV)
    assert bt.gemm_split_plan(M, N, K) == (0, 2)  # this shape takes the split-K route
    Y1, acc1 = bt.ternary_gemm(pw, q, want_acc=True)
    Y2, acc2 = bt.ternary_gemm(pw, q, want_acc=True, workspace=ws)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(acc1.cpu().numpy()[rows], ref["acc"])
    np.testing.assert_array_equal(acc2.cpu().numpy(), acc1.cpu().numpy())
    np.testing.assert_array_equal(Y1.cpu().numpy(), Y2.cpu().numpy())
    assert tol_ok(Y1.cpu().numpy()[rows], ref["Y"])


def test_gemm_rows_tail_split():
    """Row scales on the tail-split route (256 whole tiles, the last 32 split in four):
    sampled rows against the oracle, every output bit-identical to the unsplit route."""
    M, N, K, groups = 1100, 4096, 6200, [2048, 1024, 1024]
    note(f"gemm_rs tail split M={M} N={N} K={K}")
    assert bt.gemm_split_plan(M, N, K) == (256, 4)
    W = grouped(N, K, groups, 8800)
    X = synth.gaussian((M, K), 8801)
    rs = oracle.absmean_rows(W, groups)
    T = oracle.ternarize_rows(W, rs)
    Q, s, qs = oracle.quant_act(X)
    rows = np.concatenate([np.arange(3, M, 59), [M - 1]])
    acc_ref = oracle.ternary_matmul(T, Q[rows])
    pw = bt.pack_weights_rows(to_dev(W), groups)
    q = bt.quant_act(to_dev(X))
    ws = bt.gemm_workspace(M, N, K, DEV)
    Y1, acc1 = bt.ternary_gemm(pw, q, want_acc=True)
    Y2, acc2 = bt.ternary_gemm(pw, q, want_acc=True, workspace=ws)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(acc2.cpu().numpy()[rows], acc_ref)
    np.testing.assert_array_equal(acc1.cpu().numpy(), acc2.cpu().numpy())
    np.testing.assert_array_equal(Y1.cpu().numpy(), Y2.cpu().numpy())
    assert tol_ok(Y2.cpu().numpy()[rows], oracle.scale_epilogue_rows(acc_ref, rs, s[rows]))


def test_rows_group_errors():
    W = torch.zeros((10, 8), dtype=torch.float32, device=DEV)
    for bad in ([4, 5], [4, 7], [0, 10], [1] * 10):
        with pytest.raises(bt.BTError):
            bt.pack_weights_rows(W, bad)
