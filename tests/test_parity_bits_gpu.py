"""GPU parity of the 1-bit-activation path (binary W1A1 and ternary-weight W1.58A1)
against the CPU oracle: bits, scales and the int32 accumulator bit-exact, Y within
|dY| <= 1e-5 |Y| + 1e-6. The expected bit words are the oracle's signs laid out in the
documented bit order; no expected value comes from the GPU.
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


def expected_words(B, layout):
    """Bit words of the +-1 rows B (bit set for -1) in the documented layout."""
    M, K = B.shape
    per, nwords = (32, (K + 127) // 128 * 4) if layout == bt.BITS_PLAIN else (16, (K + 63) // 64 * 4)
    out = np.zeros((M, nwords), dtype=np.uint64)
    for k in range(K):
        b = k % per
        bit = b if layout == bt.BITS_PLAIN else 8 * (b % 4) + 2 * (b // 4)
        out[:, k // per] |= (B[:, k] < 0).astype(np.uint64) << np.uint64(bit)
    return out.astype(np.uint32)


def inputs(M, N, K, seed):
    W = synth.gaussian((N, K), seed, 0.02)
    X = synth.gaussian((M, K), seed + 1)
    X[:, ::7] = 0.0            # zeros binarize to +1
    X[:, 3::11] = -0.0         # and so do negative zeros
    return W, X


@pytest.mark.parametrize("layout", [1, 2])
@pytest.mark.parametrize("M,K", [(1, 1), (3, 65), (2, 129), (4, 300), (1, 4096), (16, 2560)])
def test_binarize_act(M, K, layout):
    note(f"binarize M={M} K={K} layout={layout}")
    _, X = inputs(M, 8, K, 7100 + K)
    Xb, sx = bt.binarize_act(to_dev(X), layout)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(Xb.cpu().numpy().view(np.uint32), expected_words(oracle.binarize(X), layout))
    np.testing.assert_array_equal(sx.cpu().numpy().view(np.uint32), oracle.absmax_rows(X).view(np.uint32))


@pytest.mark.parametrize("N,K", [(1, 1), (65, 129), (100, 300), (64, 128), (4096, 4096)])
def test_pack_binary(N, K):
    note(f"pack_binary N={N} K={K}")
    W, _ = inputs(1, N, K, 7200 + N + K)
    pw = bt.pack_weights_binary(to_dev(W))
    torch.cuda.synchronize()
    assert pw.scale.cpu().numpy().view(np.uint32)[0] == oracle.absmax_rows(W.reshape(1, -1)).view(np.uint32)[0]
    words = pw.data.cpu().numpy().view(np.uint32)
    KC, NB = (K + 127) // 128, (N + 63) // 64
    # word (rb, c, r, j) at index ((rb * KC + c) * 64 + r) * 4 + j holds k = 128 c + 32 j + b at
    # bit b of row n = 64 rb + r; every bit of the padded [64 NB, 128 KC] matrix is checked,
    # the padding (rows past N, k past K) clear.
    w4 = words[: NB * KC * 64 * 4].reshape(NB, KC, 64, 4)
    bits = (w4[..., None] >> np.arange(32, dtype=np.uint32)) & 1  # [rb, c, r, j, b]
    got = bits.transpose(0, 2, 1, 3, 4).reshape(NB * 64, KC * 128).astype(np.uint8)
    want = np.zeros_like(got)
    want[:N, :K] = oracle.binarize(W) < 0
    np.testing.assert_array_equal(got, want)


BITS_CASES = [(1, 1, 1), (1, 100, 300), (3, 65, 129), (4, 200, 700), (16, 130, 517), (1, 4096, 4096),
              (1, 11008, 4096), (8, 4096, 4096)]


@pytest.mark.parametrize("M,N,K", BITS_CASES)
def test_binary_gemv(M, N, K):
    note(f"binary gemv M={M} N={N} K={K}")
    W, X = inputs(M, N, K, 7300 + N + K)
    ref = oracle.binary_layer(W, X)
    pw = bt.pack_weights_binary(to_dev(W))
    Y, acc = bt.binary_gemv(pw, bt.binarize_act(to_dev(X), bt.BITS_PLAIN), want_acc=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(acc.cpu().numpy(), ref["acc"])
    assert tol_ok(Y.cpu().numpy(), ref["Y"])


@pytest.mark.parametrize("M,N,K", BITS_CASES)
def test_ternary_gemv_a1(M, N, K):
    note(f"ternary a1 gemv M={M} N={N} K={K}")
    W, X = inputs(M, N, K, 7400 + N + K)
    ref = oracle.ternary_a1_layer(W, X)
    pw = bt.pack_weights(to_dev(W))
    Y, acc = bt.ternary_gemv_a1(pw, bt.binarize_act(to_dev(X), bt.BITS_CODES), want_acc=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(acc.cpu().numpy(), ref["acc"])
    assert tol_ok(Y.cpu().numpy(), ref["Y"])


def test_bits_errors():
    W = to_dev(synth.gaussian((8, 64), 7500, 0.02))
    X = to_dev(synth.gaussian((17, 64), 7501))
    with pytest.raises(bt.BTError):  # 17 tokens: above the GEMV limit
        bt.binary_gemv(bt.pack_weights_binary(W), bt.binarize_act(X, bt.BITS_PLAIN))
    with pytest.raises(bt.BTError):  # unknown layout
        bt.binarize_act(X, 3)
