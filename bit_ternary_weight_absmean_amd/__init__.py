"""MI355X-native BitNet b1.58 W1.58A8 ternary linear layer.

The compute lives in ``libbt.so`` (hand-written HIP kernels for gfx950 behind the C ABI
of ``include/bt.h``). This module only marshals torch tensors (device memory) and the
current HIP stream into those calls; every step of the path runs in the library's
kernels. Names follow the C ABI: ``pack_weights``, ``quant_act``, ``ternary_gemv``,
``ternary_gemm`` (+ ``unpack_weights``, ``linear``, and ``pack_weights_rows`` for
row-group weight scales, which the product calls then take in place of one scale).
"""
from __future__ import annotations

from ._lib import BTError, lib
from .api import (
    BITS_CODES,
    BITS_PLAIN,
    CALL_GEMM,
    CALL_GEMM_WS,
    CALL_GEMV,
    CALL_LINEAR,
    CALL_QUANT,
    GEMV_AUTO,
    GEMV_DOT4,
    GEMV_LUT,
    GEMV_MAX_M,
    GEMV_MFMA,
    GEMV_STAGED,
    STATIC_SCRATCH_BYTES,
    PackedWeight,
    act_row_bytes,
    binarize_act,
    binary_gemv,
    gemm_split_plan,
    gemm_workspace,
    gemm_workspace_bytes,
    kernel_plan,
    linear,
    linear_static,
    linear_workspace_bytes,
    pack_weights,
    pack_weights_binary,
    pack_weights_rows,
    pack_workspace_bytes,
    packed_weight_bytes,
    quant_act,
    ternary_gemm,
    ternary_gemv,
    ternary_gemv_a1,
    unpack_weights,
)

__all__ = [
    "BITS_CODES", "BITS_PLAIN", "binarize_act", "binary_gemv", "pack_weights_binary", "ternary_gemv_a1",
    "BTError", "lib", "GEMV_AUTO", "GEMV_DOT4", "GEMV_LUT", "GEMV_MFMA", "GEMV_STAGED", "GEMV_MAX_M", "PackedWeight", "act_row_bytes",
    "gemm_split_plan", "gemm_workspace", "gemm_workspace_bytes", "linear", "linear_workspace_bytes", "pack_weights", "pack_weights_rows", "pack_workspace_bytes", "packed_weight_bytes", "quant_act", "ternary_gemm",
    "ternary_gemv", "unpack_weights", "kernel_plan", "CALL_LINEAR", "CALL_GEMV", "CALL_GEMM", "CALL_GEMM_WS", "CALL_QUANT", "linear_static", "STATIC_SCRATCH_BYTES",
]
