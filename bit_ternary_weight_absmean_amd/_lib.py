"""ctypes loader for libbt.so. Fails loudly when the library is missing: there is no
fallback implementation anywhere in this package."""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libbt.so")

# Every function declared in include/bt.h, with (restype, argtypes).
_i64, _i32, _vp, _sz = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t
SIGNATURES = {
    "bt_packed_weight_bytes": (_sz, [_i64, _i64]),
    "bt_act_row_bytes": (_i64, [_i64]),
    "bt_pack_workspace_bytes": (_sz, [_i64, _i64]),
    "bt_pack_weights": (_i32, [_vp, _i64, _i64, _vp, _vp, _vp, _vp]),
    "bt_unpack_weights": (_i32, [_vp, _i64, _i64, _vp, _vp]),
    "bt_quant_act": (_i32, [_vp, _i64, _i64, _vp, _vp, _vp, _vp]),
    "bt_ternary_gemv": (_i32, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _vp, _vp]),
    "bt_ternary_gemv_algo": (_i32, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _vp, _i32, _vp]),
    "bt_ternary_gemm": (_i32, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _vp, _vp]),
    "bt_gemm_workspace_bytes": (_sz, [_i64, _i64, _i64]),
    "bt_gemm_split_plan": (_i32, [_i64, _i64, _i64, _vp, _vp]),
    "bt_ternary_gemm_ws": (_i32, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _vp, _vp, _sz, _vp]),
    "bt_linear_workspace_bytes": (_sz, [_i64, _i64, _i64]),
    "bt_ternary_linear": (_i32, [_vp, _vp, _vp, _i64, _i64, _i64, _vp, _vp, _vp, _vp]),
    "bt_pack_weights_rows": (_i32, [_vp, _i64, _i64, _vp, _i64, _vp, _vp, _vp, _vp]),
    "bt_ternary_gemv_rs": (_i32, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _vp, _i32, _vp]),
    "bt_ternary_gemm_rs": (_i32, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _vp, _vp, _sz, _vp]),
    "bt_ternary_linear_rs": (_i32, [_vp, _vp, _vp, _i64, _i64, _i64, _vp, _vp, _vp, _vp]),
    "bt_ternary_linear_static": (_i32, [_vp, _vp, _vp, _i64, _i64, _i64, _vp, _vp, _vp]),
    "bt_binary_weight_bytes": (_sz, [_i64, _i64]),
    "bt_act_bits_row_bytes": (_i64, [_i64, _i32]),
    "bt_pack_weights_binary": (_i32, [_vp, _i64, _i64, _vp, _vp, _vp, _vp]),
    "bt_binarize_act": (_i32, [_vp, _i64, _i64, _i32, _vp, _vp, _vp]),
    "bt_binary_gemv": (_i32, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _vp, _vp]),
    "bt_ternary_gemv_a1": (_i32, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _vp, _vp]),
    "bt_kernel_plan": (_i32, [_i32, _i64, _i64, _i64, _i32, _i32, ctypes.c_char_p, _sz]),
    "bt_status_str": (ctypes.c_char_p, [_i32]),
    "bt_last_error": (ctypes.c_char_p, []),
}

_lib = None


class BTError(RuntimeError):
    def __init__(self, status: int, name: str, message: str):
        super().__init__(f"{name} ({status}): {message}")
        self.status = status
        self.name = name


def lib() -> ctypes.CDLL:
    """The loaded libbt.so. Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m bit_ternary_weight_absmean_amd.build` "
                "(there is no CPU fallback)")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(handle, name)
            f.restype = res
            f.argtypes = args
        _lib = handle
    return _lib


def check(status: int) -> None:
    if status != 0:
        L = lib()
        raise BTError(status, L.bt_status_str(status).decode(), L.bt_last_error().decode())
