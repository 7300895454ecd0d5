"""GPU parity on edge-case inputs: extreme and subnormal magnitudes, all-negative tokens,
absmax at exact powers of two times 127, subnormal weight rows under row scales, and
short or unaligned K at layer-sized N. Every route is compared with the oracle (int8
activations, their scales and sums bit-exact; acc bit-exact; Y within 1e-5 |Y| + 1e-6).

The magnitudes stay inside the contract: every token's absmax a satisfies
127 / FLT_MAX < a (so 127 / a is finite) and the outputs stay finite.
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
F32_TINY = np.float32(np.finfo(np.float32).tiny)  # smallest normal, 2^-126


def note(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def tol_ok(y, ref):
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    return bool(np.all(np.isfinite(ref))) and bool(np.all(np.abs(y - ref) <= 1e-5 * np.abs(ref) + 1e-6))


def bits(x):
    return np.asarray(x, np.float32).view(np.uint32)


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def edge_tokens(K, seed):
    """Sixteen tokens of K values, each row one edge case (a Gaussian base of the given seed
    scaled or overwritten)."""
    g = synth.gaussian((16, K), seed)
    X = np.empty((16, K), np.float32)
    big, small = np.float32(1e30), np.float32(1e-30)
    # 0: +-1e30 and +-1e-30 interleaved (the small ones quantize to 0)
    X[0] = np.where(np.arange(K) % 2 == 0, big, small) * np.sign(g[0] + 0.1).astype(np.float32)
    # 1: Gaussian with every third element subnormal (absmax normal)
    X[1] = g[1]
    X[1, ::3] = np.float32(3e-41) * np.sign(g[1, ::3] + 0.1).astype(np.float32)
    X[1, 1] = np.float32(1.4e-45)
    # 2: all negative
    X[2] = -np.abs(g[2]) - np.float32(1e-3)
    # 3: absmax exactly 127 * 2^3 (inv = 2^-3 exactly), multiples of 0.5 * 2^3 (ties of x * inv)
    X[3] = np.round(g[3] * 200) * np.float32(4.0)
    X[3, 0] = np.float32(127 * 8)
    X[3] = np.clip(X[3], -127 * 8, 127 * 8)
    # 4: absmax exactly 127 * 2^-10, the rest integer multiples of 2^-11 (ties)
    X[4] = np.clip(np.round(g[4] * 60), -254, 254) * np.float32(2.0 ** -11)
    X[4, K // 2] = -np.float32(127 * 2.0 ** -10)
    # 5: absmax 1e36 (large; outputs stay finite)
    X[5] = g[5] * np.float32(2e35)
    X[5, 0] = np.float32(1e36)
    # 6: absmax 1e-36, just above 127 / FLT_MAX (the smallest absmax the contract allows)
    X[6] = g[6] * np.float32(2e-37)
    X[6, -1] = np.float32(1e-36)
    # 7: all zero
    X[7] = 0.0
    # 8: one non-zero element
    X[8] = 0.0
    X[8, K // 3] = np.float32(-0.75)
    # 9: subnormal-scale neighbours of the smallest normal number beside a unit absmax
    X[9] = g[9] * F32_TINY
    X[9, 0] = np.float32(1.0)
    # 10: constant magnitude with alternating signs (every q = +-127)
    X[10] = np.where(np.arange(K) % 2 == 0, 3.25, -3.25).astype(np.float32)
    # 11: values at +-(n + 0.5) / inv for small n (round-half-to-even ties at absmax 127)
    X[11] = (np.round(g[11] * 20) + np.float32(0.5)).astype(np.float32)
    X[11, 0] = np.float32(127.0)
    X[11] = np.clip(X[11], -127, 127)
    # 12..15: plain Gaussian at magnitudes 1e-20, 1, 1e20 and a negative-mean mix
    X[12] = g[12] * np.float32(1e-20)
    X[13] = g[13]
    X[14] = g[14] * np.float32(1e20)
    X[15] = g[15] - np.float32(2.0)
    assert np.all(np.isfinite(X))
    return np.ascontiguousarray(X)


@pytest.mark.parametrize("K", [2560, 6912, 1000, 37])
def test_edge_tokens_quantize_bit_exact(K):
    note(f"edge tokens quant K={K}")
    X = edge_tokens(K, 5100 + K)
    Xq, sx, xsum = bt.quant_act(to_dev(X))
    torch.cuda.synchronize()
    Q, s_ref, qs_ref = oracle.quant_act(X)
    np.testing.assert_array_equal(Xq.cpu().numpy()[:, :K], Q)
    np.testing.assert_array_equal(bits(sx.cpu().numpy()), bits(s_ref))
    np.testing.assert_array_equal(xsum.cpu().numpy(), qs_ref)


@pytest.mark.parametrize("N,K", [(3840, 2560), (2560, 6912), (512, 1000), (2560, 37)])
def test_edge_tokens_every_route(N, K):
    """The edge tokens through the fused kernel (four at a time), the staged and direct
    GEMVs, the dot4 GEMV and the GEMM."""
    note(f"edge tokens products N={N} K={K}")
    X = edge_tokens(K, 5200 + K)
    W = synth.gaussian((N, K), 5300 + N + K, 0.02)
    ref = oracle.linear(W, X)
    pw = bt.pack_weights(to_dev(W))

    def check(Y, acc, rows, what):
        torch.cuda.synchronize()
        acc = acc.cpu().numpy()
        bad = np.argwhere(acc != ref["acc"][rows])
        assert bad.size == 0, f"{what}: {len(bad)} acc mismatches, first {bad[:5].tolist()}"
        assert tol_ok(Y.cpu().numpy(), ref["Y"][rows]), f"{what}: Y outside tolerance"

    for m0 in range(0, 16, 4):
        rows = slice(m0, m0 + 4)
        if bt.linear_workspace_bytes(4, N, K) == 0:
            Y, acc = bt.linear(to_dev(X[rows]), pw, want_acc=True)
            check(Y, acc, rows, f"fused tokens {m0}..{m0 + 3}")
        q = bt.quant_act(to_dev(X[rows]))
        Y, acc = bt.ternary_gemv(pw, q, want_acc=True, algo=bt.GEMV_DOT4)
        check(Y, acc, rows, f"dot4 tokens {m0}..{m0 + 3}")
    q = bt.quant_act(to_dev(X))
    for algo, what in ((bt.GEMV_STAGED, "staged"), (bt.GEMV_MFMA, "direct")):
        Y, acc = bt.ternary_gemv(pw, q, want_acc=True, algo=algo)
        check(Y, acc, slice(0, 16), what)
    Y, acc = bt.ternary_gemm(pw, q, want_acc=True)
    check(Y, acc, slice(0, 16), "gemm")
    Y, acc = bt.linear(to_dev(X), pw, want_acc=True)
    check(Y, acc, slice(0, 16), "linear, 16 tokens")


def subnormal_rows_matrix(N, K, seed):
    """Weights whose rows have very different magnitudes: subnormal rows (integer multiples
    of 2^-146 and of 2^-149), a row at the smallest normal scale, zero rows and Gaussian rows."""
    W = synth.gaussian((N, K), seed, 0.02)
    ints = np.round(synth.gaussian((N, K), seed + 1) * 2).astype(np.float32)
    W[0] = ints[0] * np.float32(2.0 ** -146)          # subnormal row, gamma subnormal
    W[1] = ints[1] * np.float32(2.0 ** -149)          # multiples of the smallest subnormal
    W[2] = W[2] * np.float32(2.0 ** -120)             # near the smallest normal
    W[3] = 0.0                                         # zero row: scale 0, every code 0
    W[4, : K // 2] = ints[4, : K // 2] * np.float32(2.0 ** -140)  # half subnormal, half Gaussian
    W[5] = ints[5] * np.float32(2.0 ** -147)
    W[5, 0] = np.float32(2.0 ** -126)                  # one normal element in a subnormal row
    return np.ascontiguousarray(W)


@pytest.mark.parametrize("N,K", [(64, 256), (2560, 2560), (70, 1001)])
def test_subnormal_weight_rows_row_scales(N, K):
    """One group per row (bt_pack_weights_rows with no groups): subnormal row scales, whose
    halving rounds in fp32, take the same codes on both sides; products on every route."""
    note(f"subnormal weight rows N={N} K={K}")
    W = subnormal_rows_matrix(N, K, 5400 + N)
    X = synth.gaussian((4, K), 5500 + K)
    ref = oracle.linear_rows(W, X, None)
    rs_ref = oracle.absmean_rows(W, None)
    assert rs_ref[0] < F32_TINY and rs_ref[1] < F32_TINY  # the case under test: subnormal scales
    pw = bt.pack_weights_rows(to_dev(W), None)
    T = bt.unpack_weights(pw)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(pw.scale.cpu().numpy()), bits(rs_ref))
    np.testing.assert_array_equal(T.cpu().numpy(), oracle.ternarize_rows(W, rs_ref))
    for what, fn in (("linear", lambda: bt.linear(to_dev(X), pw, want_acc=True)),
                     ("staged", lambda: bt.ternary_gemv(pw, bt.quant_act(to_dev(X)), want_acc=True,
                                                        algo=bt.GEMV_STAGED)),
                     ("gemm", lambda: bt.ternary_gemm(pw, bt.quant_act(to_dev(X)), want_acc=True))):
        Y, acc = fn()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(acc.cpu().numpy(), ref["acc"], err_msg=what)
        assert tol_ok(Y.cpu().numpy(), ref["Y"]), what


def test_subnormal_matrix_one_scale():
    """A whole matrix of subnormal weights (one scale per matrix, gamma subnormal)."""
    note("subnormal matrix")
    N, K = 300, 700
    W = (np.round(synth.gaussian((N, K), 5600) * 2) * np.float32(2.0 ** -145)).astype(np.float32)
    X = synth.gaussian((3, K), 5601)
    ref = oracle.linear(W, X)
    assert ref["gamma"] < F32_TINY
    pw = bt.pack_weights(to_dev(W))
    torch.cuda.synchronize()
    assert bits(pw.scale.cpu().numpy())[0] == bits(ref["gamma"])
    np.testing.assert_array_equal(bt.unpack_weights(pw).cpu().numpy(), ref["T"])
    Y, acc = bt.linear(to_dev(X), pw, want_acc=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(acc.cpu().numpy(), ref["acc"])
    assert tol_ok(Y.cpu().numpy(), ref["Y"])


SHORT_K = [1, 2, 3, 4, 5, 7, 13, 31, 33, 63, 65, 127, 255, 257, 2561, 2563]


@pytest.mark.parametrize("K", SHORT_K)
@pytest.mark.parametrize("N", [2560, 3840])
def test_short_and_unaligned_k_at_layer_n(N, K):
    """K = 1..63 and K % 4 != 0 at layer-sized N, through every route."""
    note(f"short K N={N} K={K}")
    W = synth.gaussian((N, K), 5700 + N + K, 0.02)
    X = synth.gaussian((40, K), 5800 + K)
    X[1] = 0.0
    ref = oracle.linear(W, X)
    pw = bt.pack_weights(to_dev(W))
    outs = []
    for M in (1, 3, 4):
        if bt.linear_workspace_bytes(M, N, K) == 0:
            outs.append((f"fused M={M}", M, bt.linear(to_dev(X[:M]), pw, want_acc=True)))
        outs.append((f"dot4 M={M}", M, bt.ternary_gemv(pw, bt.quant_act(to_dev(X[:M])), want_acc=True,
                                                       algo=bt.GEMV_DOT4)))
    q16 = bt.quant_act(to_dev(X[:16]))
    outs.append(("staged M=16", 16, bt.ternary_gemv(pw, q16, want_acc=True, algo=bt.GEMV_STAGED)))
    outs.append(("direct M=16", 16, bt.ternary_gemv(pw, q16, want_acc=True, algo=bt.GEMV_MFMA)))
    outs.append(("linear M=40", 40, bt.linear(to_dev(X), pw, want_acc=True)))
    outs.append(("gemm M=40", 40, bt.ternary_gemm(pw, bt.quant_act(to_dev(X)), want_acc=True)))
    torch.cuda.synchronize()
    for what, M, (Y, acc) in outs:
        np.testing.assert_array_equal(acc.cpu().numpy(), ref["acc"][:M], err_msg=what)
        assert tol_ok(Y.cpu().numpy(), ref["Y"][:M]), what
