"""The C ABI without a GPU: the library loads, exports every function include/bt.h
declares, sizes its buffers as documented, and rejects bad arguments on the host
before any HIP call (so these run on a CPU-only machine)."""
import ctypes
import os
import re

import pytest

import bit_ternary_weight_absmean_amd as bt
from bit_ternary_weight_absmean_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bt.h")

BT_OK, BT_ERR_NULL, BT_ERR_SHAPE, BT_ERR_UNSUPPORTED, BT_ERR_ALIGN, BT_ERR_HIP = range(6)
FAKE = 0x10000  # an aligned, never-dereferenced address: every call below fails validation first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bt_[a-z0-9_]+)\s*\(", text)))


def test_header_and_binding_agree():
    assert declared_functions() == sorted(_lib.SIGNATURES)


def test_library_exports_every_declared_symbol():
    L = bt.lib()
    for name in declared_functions():
        assert hasattr(L, name), name


def test_built_for_gfx950():
    data = open(_lib.LIB_PATH, "rb").read()
    assert b"gfx950" in data


def test_sizes():
    L = bt.lib()
    assert L.bt_packed_weight_bytes(512, 256) == 512 * 256 // 4
    assert L.bt_packed_weight_bytes(3840, 2560) == 2_457_600
    assert L.bt_packed_weight_bytes(57344, 8192) == 117_440_512
    assert L.bt_packed_weight_bytes(100, 300) == 128 * 320 // 4  # padded to 64 x 64
    assert L.bt_packed_weight_bytes(0, 300) == 0
    assert L.bt_act_row_bytes(2560) == 2560
    assert L.bt_act_row_bytes(300) == 512
    assert L.bt_act_row_bytes(1) == 256
    assert L.bt_act_row_bytes(6912) == 6912
    assert L.bt_act_row_bytes(0) == 0
    assert L.bt_pack_workspace_bytes(3, 5) == 256
    assert L.bt_pack_workspace_bytes(100, 5) == 1024


def test_gemm_split_plan():
    """The GEMM's work split (host logic): whole tiles, tail split, split of every tile, and
    the workspace bytes that follow from it."""
    def plan(M, N, K):
        full, splits = ctypes.c_int64(-1), ctypes.c_int32(-1)
        assert bt.lib().bt_gemm_split_plan(M, N, K, ctypes.byref(full), ctypes.byref(splits)) == BT_OK
        return full.value, splits.value

    def ws_bytes(M, N, full, splits):
        tiles = -(-M // 64) * -(-N // 256)
        if splits == 1:
            return 0
        n = tiles - full
        return -(-4 * n // 256) * 256 + n * splits * 64 * 256 * 4

    cases = {
        # 2B prefill at M = 2048: 480, 320 and 1728 tiles of 20 steps stay whole; down
        # (320 tiles of 54 steps) computes 256 whole and splits the last 64 in four.
        (2048, 3840, 2560): (480, 1), (2048, 2560, 2560): (320, 1), (2048, 13824, 2560): (1728, 1),
        (2048, 2560, 6912): (256, 4),
        (4096, 2560, 6912): (512, 2),   # 640 tiles: the last 128 in two
        (1024, 13824, 2560): (864, 1),  # tail of 96 tiles, but shares of 10 steps: whole
        # at most two 64 x 64 tiles per CU (512) and K >= 512: the small-M form, no split
        (256, 3840, 2560): (60, 1), (256, 2560, 6912): (40, 1), (100, 2500, 6900): (20, 1),
        (70, 600, 2500): (6, 1), (65, 300, 1600): (4, 1), (256, 4096, 512): (64, 1),
        (520, 2500, 6900): (90, 1), (300, 3500, 2600): (70, 1), (512, 3840, 2560): (120, 1),
        # more 64 x 64 tiles, few 64 x 256 ones: every tile split
        (600, 3500, 6900): (0, 4), (650, 3300, 5500): (0, 3), (700, 3000, 4000): (0, 2),
        (1024, 2560, 6912): (0, 4), (256, 13824, 2560): (216, 1), (70, 600, 500): (6, 1),
        (1100, 4096, 6200): (256, 4), (250, 22700, 3100): (256, 2),
        (5, 5, 0): (1, 1), (0, 5, 5): (0, 1),
    }
    for (M, N, K), want in cases.items():
        assert plan(M, N, K) == want, (M, N, K)
        assert bt.lib().bt_gemm_workspace_bytes(M, N, K) == ws_bytes(M, N, *want), (M, N, K)
    # which kernel each form runs
    for (M, N, K), kern in {(256, 3840, 2560): "k_gemm_ks<NS=3,ROWS=0>", (256, 4096, 512): "k_gemm_ks<NS=3,ROWS=0>",
                            (256, 4160, 512): "k_gemm_ks<NS=2,ROWS=0>", (512, 4096, 512): "k_gemm_ks<NS=2,ROWS=0>",
                            (520, 4160, 512): "k_gemm<SPLITK=0", (256, 3840, 511): "k_gemm<SPLITK=0",
                            (650, 3300, 5500): "k_gemm<SPLITK=1"}.items():
        assert bt.kernel_plan(bt.CALL_GEMM_WS, M, N, K).startswith(kern), (M, N, K)
    full, splits = ctypes.c_int64(), ctypes.c_int32()
    assert bt.lib().bt_gemm_split_plan(-1, 5, 5, ctypes.byref(full), ctypes.byref(splits)) == BT_ERR_SHAPE
    assert bt.lib().bt_gemm_split_plan(5, 5, 5, None, ctypes.byref(splits)) == BT_ERR_NULL


def _gemv(L, *, Wp=FAKE, ws=FAKE, Xq=FAKE, sx=FAKE, xsum=FAKE, M=1, N=64, K=64, Y=FAKE, acc=0, algo=0):
    return L.bt_ternary_gemv_algo(Wp, ws, Xq, sx, xsum, M, N, K, Y, acc, algo, None)


def test_product_validation():
    L = bt.lib()
    assert _gemv(L, Y=0, acc=0) == BT_ERR_NULL
    assert _gemv(L, Wp=0) == BT_ERR_NULL
    assert _gemv(L, xsum=0) == BT_ERR_NULL
    assert _gemv(L, M=-1) == BT_ERR_SHAPE
    assert _gemv(L, K=-5) == BT_ERR_SHAPE
    assert _gemv(L, K=131073) == BT_ERR_SHAPE
    assert _gemv(L, M=17) == BT_ERR_UNSUPPORTED
    assert _gemv(L, M=5, algo=1) == BT_ERR_UNSUPPORTED
    assert _gemv(L, algo=7) == BT_ERR_UNSUPPORTED
    assert _gemv(L, Wp=FAKE + 4) == BT_ERR_ALIGN
    assert _gemv(L, Xq=FAKE + 8) == BT_ERR_ALIGN
    assert _gemv(L, Y=FAKE + 2) == BT_ERR_ALIGN
    assert b"Y and acc" in _reason(L, lambda: _gemv(L, Y=0, acc=0))
    # M == 0 or N == 0 is a no-op that succeeds without touching the device
    assert _gemv(L, M=0) == BT_OK
    assert _gemv(L, N=0) == BT_OK
    assert L.bt_ternary_gemm(FAKE, FAKE, FAKE, FAKE, FAKE, 0, 64, 64, FAKE, 0, None) == BT_OK
    assert L.bt_ternary_gemm(FAKE, FAKE, FAKE, FAKE, FAKE, 3, 64, 64, 0, 0, None) == BT_ERR_NULL
    assert L.bt_ternary_gemm(FAKE + 1, FAKE, FAKE, FAKE, FAKE, 3, 64, 64, FAKE, 0, None) == BT_ERR_ALIGN


def _reason(L, call):
    call()
    return L.bt_last_error()


def test_pack_and_quant_validation():
    L = bt.lib()
    assert L.bt_pack_weights(FAKE, 4, 4, FAKE, 0, FAKE, None) == BT_ERR_NULL
    assert L.bt_pack_weights(0, 4, 4, FAKE, FAKE, FAKE, None) == BT_ERR_NULL
    assert L.bt_pack_weights(FAKE, 4, 4, FAKE, FAKE, 0, None) == BT_ERR_NULL
    assert L.bt_pack_weights(FAKE, -1, 4, FAKE, FAKE, FAKE, None) == BT_ERR_SHAPE
    assert L.bt_pack_weights(FAKE + 4, 4, 4, FAKE, FAKE, FAKE, None) == BT_ERR_ALIGN
    assert L.bt_pack_weights(FAKE, 4, 4, FAKE, FAKE, FAKE + 4, None) == BT_ERR_ALIGN
    assert L.bt_unpack_weights(0, 4, 4, FAKE, None) == BT_ERR_NULL
    assert L.bt_unpack_weights(FAKE, 0, 4, 0, None) == BT_OK
    assert L.bt_quant_act(FAKE, -2, 4, FAKE, FAKE, FAKE, None) == BT_ERR_SHAPE
    assert L.bt_quant_act(FAKE, 2, 4, FAKE, 0, FAKE, None) == BT_ERR_NULL
    assert L.bt_quant_act(FAKE, 2, 4, FAKE + 4, FAKE, FAKE, None) == BT_ERR_ALIGN
    assert L.bt_quant_act(FAKE + 2, 2, 4, FAKE, FAKE, FAKE, None) == BT_ERR_ALIGN
    assert L.bt_quant_act(FAKE, 0, 4, 0, 0, 0, None) == BT_OK


def test_shape_limits():
    """M, N <= 2^23, N * K and M * N <= 2^36: larger shapes fail on the host (every launch
    then fits 2^32 work-items)."""
    L = bt.lib()
    big, over = 1 << 23, (1 << 23) + 1
    assert L.bt_quant_act(FAKE, over, 4, FAKE, FAKE, FAKE, None) == BT_ERR_SHAPE
    assert L.bt_pack_weights(FAKE, over, 4, FAKE, FAKE, FAKE, None) == BT_ERR_SHAPE
    assert L.bt_pack_weights(FAKE, big, 1 << 17, FAKE, FAKE, FAKE, None) == BT_ERR_SHAPE  # N * K = 2^40
    assert L.bt_unpack_weights(FAKE, big, 1 << 17, FAKE, None) == BT_ERR_SHAPE
    assert L.bt_pack_weights_binary(FAKE, big, 1 << 17, FAKE, FAKE, FAKE, None) == BT_ERR_SHAPE
    assert _gemv(L, N=over) == BT_ERR_SHAPE
    # M * N = 2^37 fails; 2^36 passes the shape checks (and then fails on the NULL acc/Y pair)
    assert L.bt_ternary_gemm(FAKE, FAKE, FAKE, FAKE, FAKE, big, 1 << 14, 64, FAKE, 0, None) == BT_ERR_SHAPE
    assert L.bt_ternary_gemm(FAKE, FAKE, FAKE, FAKE, FAKE, big, 1 << 13, 64, 0, 0, None) == BT_ERR_NULL
    assert b"2^36" in _reason(L, lambda: L.bt_ternary_gemm(FAKE, FAKE, FAKE, FAKE, FAKE, big, 1 << 14, 64, FAKE, 0,
                                                           None))
    assert L.bt_ternary_linear(FAKE, FAKE, FAKE, over, 64, 64, FAKE, 0, FAKE, None) == BT_ERR_SHAPE
    # the linear layer refuses before its quantizer launch, so nothing is enqueued
    assert L.bt_ternary_linear(FAKE, FAKE, FAKE, big, 1 << 14, 64, FAKE, 0, FAKE, None) == BT_ERR_SHAPE
    assert L.bt_gemm_workspace_bytes(over, 64, 64) == 0


def test_status_strings():
    L = bt.lib()
    names = [L.bt_status_str(i).decode() for i in range(6)]
    assert names == ["BT_OK", "BT_ERR_NULL", "BT_ERR_SHAPE", "BT_ERR_UNSUPPORTED", "BT_ERR_ALIGN", "BT_ERR_HIP"]
    assert L.bt_status_str(99).decode() == "BT_ERR_UNKNOWN"


def test_python_error_type():
    with pytest.raises(bt.BTError) as e:
        _lib.check(BT_ERR_SHAPE)
    assert e.value.name == "BT_ERR_SHAPE"


def test_product_path_has_no_oracle_or_fallback():
    """The package never imports the oracle, and its sources name no CPU fallback."""
    pkg = os.path.dirname(bt.__file__)
    for fn in os.listdir(pkg):
        if fn.endswith(".py"):
            src = open(os.path.join(pkg, fn)).read()
            assert "import oracle" not in src and "from oracle" not in src, fn
