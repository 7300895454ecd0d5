"""The Python wrapper rejects buffers the library would read or write out of bounds
(wrong shape, dtype, size, layout or device) with a Python error, before any call into
libbt.so. Runs on the CPU: the device check is relaxed for CPU tensors so that every
other check is reached, and none of these calls gets as far as the library."""
import pytest
import torch

import bit_ternary_weight_absmean_amd as bt
from bit_ternary_weight_absmean_amd import api

CPU = torch.device("cpu")


@pytest.fixture
def host_ok(monkeypatch):
    """Treat CPU tensors as device tensors (so the checks after the device check run), and
    fail the test if any call reaches the library's launch entry points."""
    monkeypatch.setattr(api, "_on_device", lambda t: True)

    class NoLaunch:
        def __init__(self, real):
            self._real = real

        def __getattr__(self, name):
            if name.endswith("_bytes") or name.endswith("_row_bytes") or name in ("bt_status_str", "bt_last_error"):
                return getattr(self._real, name)
            raise AssertionError(f"{name} was called with arguments the wrapper should have rejected")

    real = bt.lib()
    monkeypatch.setattr(api, "lib", lambda: NoLaunch(real))


def packed(N, K, rows=False):
    data = torch.zeros(max(bt.packed_weight_bytes(N, K), 16), dtype=torch.uint8)
    scale = torch.zeros(N if rows else 1, dtype=torch.float32)
    return bt.PackedWeight(data, scale, N, K, row_scales=rows)


def quant(M, K):
    return (torch.zeros((M, bt.act_row_bytes(K)), dtype=torch.int8), torch.zeros(M, dtype=torch.float32),
            torch.zeros(M, dtype=torch.int32))


def test_cpu_tensors_are_rejected_without_relaxation():
    pw = packed(64, 256)
    with pytest.raises(ValueError, match="device tensor"):
        bt.ternary_gemv(pw, quant(1, 256))
    with pytest.raises(ValueError, match="device tensor"):
        bt.quant_act(torch.zeros((1, 256)))


def test_product_rejects_bad_activations(host_ok):
    pw = packed(64, 300)
    Xq, sx, xs = quant(2, 300)
    with pytest.raises(ValueError, match="Xq must have shape"):
        bt.ternary_gemv(pw, (Xq[:, :300].contiguous(), sx, xs))  # rows not padded to 512
    with pytest.raises(ValueError, match="Xq must have shape"):
        bt.ternary_gemv(pw, quant(2, 256))  # quantized for another K
    with pytest.raises(TypeError, match="Xq must be"):
        bt.ternary_gemv(pw, (Xq.to(torch.uint8), sx, xs))
    with pytest.raises(ValueError, match="x_sum must have shape"):
        bt.ternary_gemv(pw, (Xq, sx, xs[:1]))
    with pytest.raises(ValueError, match="s_x must have shape|Xq must have shape"):
        bt.ternary_gemm(pw, (Xq, torch.zeros(3), xs))
    with pytest.raises(TypeError, match="x_sum must be"):
        bt.ternary_gemm(pw, (Xq, sx, xs.float()))
    with pytest.raises(ValueError, match="contiguous"):
        big = torch.zeros((2, 2 * bt.act_row_bytes(300)), dtype=torch.int8)
        bt.ternary_gemv(pw, (big[:, ::2], sx, xs))


def test_product_rejects_bad_outputs(host_ok):
    pw = packed(64, 256)
    q = quant(3, 256)
    with pytest.raises(ValueError, match="out_y must have shape"):
        bt.ternary_gemv(pw, q, out_y=torch.zeros((3, 63)))
    with pytest.raises(TypeError, match="out_y must be"):
        bt.ternary_gemm(pw, q, out_y=torch.zeros((3, 64), dtype=torch.float64))
    with pytest.raises(ValueError, match="out_acc must have shape"):
        bt.ternary_gemv(pw, q, want_acc=True, out_acc=torch.zeros((64, 3), dtype=torch.int32))
    with pytest.raises(TypeError, match="out_acc must be"):
        bt.ternary_gemm(pw, q, out_acc=torch.zeros((3, 64), dtype=torch.int64))
    with pytest.raises(ValueError, match="contiguous"):
        bt.ternary_gemv(pw, q, out_y=torch.zeros((64, 3)).t())
    with pytest.raises(ValueError, match="needs Y or acc"):
        bt.ternary_gemv(pw, q, want_y=False, want_acc=False)


def test_product_rejects_short_weights(host_ok):
    pw = packed(64, 256)
    short = bt.PackedWeight(pw.data[:1000], pw.scale, 64, 256)
    with pytest.raises(ValueError, match="packed weights holds"):
        bt.ternary_gemv(short, quant(1, 256))
    rows = packed(64, 256, rows=True)
    bad = bt.PackedWeight(rows.data, rows.scale[:10], 64, 256, row_scales=True)
    with pytest.raises(ValueError, match="weight scale must have shape"):
        bt.ternary_gemm(bad, quant(1, 256))


def test_linear_rejects_small_workspace_and_bad_buffers(host_ok):
    M, N, K = 8, 4096, 4096  # the workspace route (M * K > 32768)
    need = bt.linear_workspace_bytes(M, N, K)
    assert need > 0
    pw = packed(N, K)
    X = torch.zeros((M, K))
    with pytest.raises(ValueError, match="workspace holds"):
        bt.linear(X, pw, workspace=torch.zeros(need - 1, dtype=torch.uint8))
    with pytest.raises(ValueError, match="X has K"):
        bt.linear(torch.zeros((M, K + 4)), pw)
    with pytest.raises(ValueError, match=r"X must be \[M, K\]"):
        bt.linear(torch.zeros(K), pw)
    with pytest.raises(ValueError, match="out_y must have shape"):
        bt.linear(X, pw, out_y=torch.zeros((M, N - 1)))
    with pytest.raises(TypeError, match="X must be"):
        bt.linear(X.double(), pw)


def test_quant_act_rejects_bad_out(host_ok):
    X = torch.zeros((2, 300))
    Xq, sx, xs = quant(2, 300)
    with pytest.raises(ValueError, match="Xq must have shape"):
        bt.quant_act(X, out=(Xq[:1].contiguous(), sx, xs))
    with pytest.raises(ValueError, match="x_sum must have shape"):
        bt.quant_act(X, out=(Xq, sx, torch.zeros(1, dtype=torch.int32)))


def test_pack_rejects_small_workspace(host_ok):
    W = torch.zeros((100, 64))
    need = bt.pack_workspace_bytes(100, 64)
    for fn in (bt.pack_weights, bt.pack_weights_rows, bt.pack_weights_binary):
        with pytest.raises(ValueError, match="workspace holds"):
            fn(W, workspace=torch.zeros(need - 8, dtype=torch.uint8))


def test_bits_products_reject_bad_buffers(host_ok):
    N, K = 64, 300
    pw = packed(N, K)
    words = bt.lib().bt_act_bits_row_bytes(K, bt.BITS_CODES) // 4
    good = (torch.zeros((2, words), dtype=torch.int32), torch.zeros(2))
    with pytest.raises(ValueError, match="Xb must have shape"):
        bt.ternary_gemv_a1(pw, (good[0][:, :1].contiguous(), good[1]))
    with pytest.raises(TypeError, match="x_scale must be"):
        bt.ternary_gemv_a1(pw, (good[0], torch.zeros(2, dtype=torch.float64)))
    binw = bt.PackedWeight(torch.zeros(16, dtype=torch.uint8), torch.zeros(1), N, K)
    with pytest.raises(ValueError, match="packed weights holds"):
        bt.binary_gemv(binw, good)
