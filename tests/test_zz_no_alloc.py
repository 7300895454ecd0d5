"""bt_ternary_linear_static (the entry point that allocates nothing and takes no workspace)
against bt_ternary_linear with a caller workspace: bit-identical acc and Y, on calls in a
row whose inputs shrink (so the static scratch holds the previous call's larger contents),
through every route that uses scratch (quantizer + GEMM with split-K counters, quantizer +
GEMV) and the fused one that does not. Calls go through the C ABI with caller-allocated
outputs."""
import ctypes
import sys

import numpy as np
import pytest
import torch

import oracle
import bit_ternary_weight_absmean_amd as bt
from bit_ternary_weight_absmean_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
BT_ERR_SHAPE, BT_ERR_UNSUPPORTED = 2, 3


def note(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def call_static(pw, X, Y, acc):
    """bt_ternary_linear_static through the C ABI (raw pointers, the current stream)."""
    M, K = X.shape
    return bt.lib().bt_ternary_linear_static(pw.data.data_ptr(), pw.scale.data_ptr(), X.data_ptr(), M, pw.N, K,
                                             Y.data_ptr(), acc.data_ptr(),
                                             torch.cuda.current_stream().cuda_stream)


# Consecutive calls, each smaller than the one before: quantizer + tail-split GEMM (the
# split-K arrival counters live in the scratch), quantizer + split-K GEMM, quantizer +
# staged GEMV, the fused kernel (no scratch), quantizer + direct GEMV.
SEQUENCE = [(2048, 2560, 6912), (300, 2560, 6912), (100, 2500, 6900), (40, 700, 1000), (8, 4096, 4096),
            (1, 3840, 2560), (16, 600, 8448)]


def test_static_matches_workspace_entry_point():
    for i, (M, N, K) in enumerate(SEQUENCE):
        note(f"static linear call {i}: M={M} N={N} K={K} plan={bt.kernel_plan(bt.CALL_LINEAR, M, N, K)}")
        assert bt.linear_workspace_bytes(M, N, K) <= bt.STATIC_SCRATCH_BYTES
        W = synth.gaussian((N, K), 6100 + i, 0.02)
        X = torch.from_numpy(synth.gaussian((M, K), 6200 + i)).to(DEV)
        pw = bt.pack_weights(torch.from_numpy(W).to(DEV))
        Y_ws, acc_ws = bt.linear(X, pw, want_acc=True)
        Y = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
        acc = torch.full((M, N), -1, dtype=torch.int32, device=DEV)
        assert call_static(pw, X, Y, acc) == 0, bt.lib().bt_last_error().decode()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(acc.cpu().numpy(), acc_ws.cpu().numpy())
        np.testing.assert_array_equal(Y.cpu().numpy().view(np.uint32), Y_ws.cpu().numpy().view(np.uint32))
        if M * N * K <= 2e9:  # the oracle too, where it is quick
            ref = oracle.linear(W, X.cpu().numpy())
            np.testing.assert_array_equal(acc.cpu().numpy(), ref["acc"])
            y, r = Y.cpu().numpy().astype(np.float64), ref["Y"].astype(np.float64)
            assert np.all(np.abs(y - r) <= 1e-5 * np.abs(r) + 1e-6)


def test_static_rejects_oversized_and_bad_shapes():
    note("static linear limits")
    pw = bt.pack_weights(torch.zeros((64, 64), dtype=torch.float32, device=DEV))
    X = torch.zeros((1, 64), dtype=torch.float32, device=DEV)
    Y = torch.zeros((1, 64), dtype=torch.float32, device=DEV)
    L = bt.lib()
    # 8192 tokens of 16384 int8 columns need 128 MiB of scratch: refused on the host
    M, N, K = 8192, 64, 16384
    assert bt.linear_workspace_bytes(M, N, K) > bt.STATIC_SCRATCH_BYTES
    assert L.bt_ternary_linear_static(pw.data.data_ptr(), pw.scale.data_ptr(), X.data_ptr(), M, N, K, Y.data_ptr(),
                                      0, 0) == BT_ERR_UNSUPPORTED
    assert b"scratch" in L.bt_last_error()
    assert L.bt_ternary_linear_static(pw.data.data_ptr(), pw.scale.data_ptr(), X.data_ptr(), -1, N, K, Y.data_ptr(),
                                      0, 0) == BT_ERR_SHAPE
    with pytest.raises(ValueError):
        bt.linear_static(X, bt.pack_weights_rows(torch.zeros((64, 64), dtype=torch.float32, device=DEV)))
