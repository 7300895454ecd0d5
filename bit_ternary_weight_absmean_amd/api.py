"""Torch-facing wrappers over the C ABI (argument marshalling only).

Every function takes and returns torch tensors on a HIP device, passes raw device
pointers and ``torch.cuda.current_stream().cuda_stream`` to libbt.so, and checks the
returned status. Nothing here computes any part of the method.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass

import torch

from ._lib import check, lib

GEMV_AUTO, GEMV_DOT4, GEMV_MFMA, GEMV_LUT, GEMV_STAGED = 0, 1, 2, 3, 4
GEMV_MAX_M = 16


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _ptr(t) -> int:
    return 0 if t is None else t.data_ptr()


def _on_device(t: torch.Tensor) -> bool:
    return t.is_cuda


def _need(t: torch.Tensor, name: str, dtype: torch.dtype, shape=None, device=None):
    """Reject a tensor the library would read or write out of bounds: wrong dtype, shape
    (None: any), layout or device. Checked before any call, so a bad buffer is a Python
    error and never a device fault."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if not _on_device(t):
        raise ValueError(f"{name} must be a device tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, the weights on {device}")


def _need_bytes(t: torch.Tensor, name: str, nbytes: int, device=None):
    """A contiguous device buffer of at least ``nbytes`` bytes (any dtype)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    have = t.numel() * t.element_size()
    if have < nbytes:
        raise ValueError(f"{name} holds {have} bytes, the call needs {nbytes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if not _on_device(t):
        raise ValueError(f"{name} must be a device tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, the weights on {device}")


def _outputs(M, N, dev, want_y, want_acc, out_y, out_acc):
    """The (Y, acc) buffers of a product: the caller's (checked) or new ones."""
    if out_y is not None:
        _need(out_y, "out_y", torch.float32, (M, N), dev)
        Y = out_y
    else:
        Y = torch.empty((M, N), dtype=torch.float32, device=dev) if want_y else None
    if out_acc is not None:
        _need(out_acc, "out_acc", torch.int32, (M, N), dev)
        acc = out_acc
    else:
        acc = torch.empty((M, N), dtype=torch.int32, device=dev) if want_acc else None
    if Y is None and acc is None:
        raise ValueError("a product needs Y or acc (want_y / want_acc / out_y / out_acc)")
    return Y, acc


def _check_q(q, K: int, dev):
    """(Xq, s_x, x_sum) as bt_quant_act writes them for K input features."""
    Xq, sx, xsum = q
    if not isinstance(sx, torch.Tensor) or sx.dim() != 1:
        raise ValueError("s_x must be a 1-D tensor of M scales")
    M = sx.shape[0]
    _need(Xq, "Xq", torch.int8, (M, act_row_bytes(K)), dev)
    _need(sx, "s_x", torch.float32, (M,), dev)
    _need(xsum, "x_sum", torch.int32, (M,), dev)
    return M


def packed_weight_bytes(N: int, K: int) -> int:
    return int(lib().bt_packed_weight_bytes(N, K))


def act_row_bytes(K: int) -> int:
    return int(lib().bt_act_row_bytes(K))


def pack_workspace_bytes(N: int, K: int) -> int:
    return int(lib().bt_pack_workspace_bytes(N, K))


@dataclass
class PackedWeight:
    """A 2-bit packed ternary weight matrix and its absmean scale(s) (both on device)."""

    data: torch.Tensor   # uint8 [packed_weight_bytes(N, K)]
    scale: torch.Tensor  # float32 [1] gamma, or [N] row scales when row_scales
    N: int
    K: int
    row_scales: bool = False

    def check(self, packed_bytes: int | None = None):
        """The buffers hold what the library reads for an N x K matrix."""
        _need_bytes(self.data, "packed weights", packed_weight_bytes(self.N, self.K) if packed_bytes is None
                    else packed_bytes)
        _need(self.scale, "weight scale", torch.float32, (max(self.N, 1),) if self.row_scales else (1,),
              self.data.device)


def pack_weights(W: torch.Tensor, workspace: torch.Tensor | None = None) -> PackedWeight:
    """bt_pack_weights: absmean ternarization + 2-bit packing of W [N,K] fp32."""
    _need(W, "W", torch.float32)
    N, K = W.shape
    dev = W.device
    data = torch.empty(max(packed_weight_bytes(N, K), 16), dtype=torch.uint8, device=dev)
    scale = torch.empty(1, dtype=torch.float32, device=dev)
    ws_bytes = pack_workspace_bytes(N, K)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 8), dtype=torch.uint8, device=dev)
    else:
        _need_bytes(workspace, "workspace", ws_bytes, dev)
    check(lib().bt_pack_weights(_ptr(W), N, K, _ptr(data), _ptr(scale), _ptr(workspace), _stream(dev)))
    return PackedWeight(data, scale, N, K)


def pack_weights_rows(W: torch.Tensor, group_rows=None, workspace: torch.Tensor | None = None) -> PackedWeight:
    """bt_pack_weights_rows: packing with row-group scales (``group_rows``: the rows of each
    group in order, summing to N; None: one group per row). The result carries N row scales."""
    _need(W, "W", torch.float32)
    N, K = W.shape
    dev = W.device
    data = torch.empty(max(packed_weight_bytes(N, K), 16), dtype=torch.uint8, device=dev)
    scale = torch.empty(max(N, 1), dtype=torch.float32, device=dev)
    ws_bytes = pack_workspace_bytes(N, K)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 8), dtype=torch.uint8, device=dev)
    else:
        _need_bytes(workspace, "workspace", ws_bytes, dev)
    if group_rows is None:
        groups, ngroups = 0, 0
    else:
        arr = (ctypes.c_int64 * len(group_rows))(*[int(r) for r in group_rows])
        groups, ngroups = ctypes.cast(arr, ctypes.c_void_p).value, len(group_rows)
    check(lib().bt_pack_weights_rows(_ptr(W), N, K, groups, ngroups, _ptr(data), _ptr(scale), _ptr(workspace),
                                     _stream(dev)))
    return PackedWeight(data, scale, N, K, row_scales=True)


def unpack_weights(pw: PackedWeight) -> torch.Tensor:
    """bt_unpack_weights: the ternary codes t in {-1,0,1} as int8 [N,K]."""
    pw.check()
    T = torch.empty((pw.N, pw.K), dtype=torch.int8, device=pw.data.device)
    check(lib().bt_unpack_weights(_ptr(pw.data), pw.N, pw.K, _ptr(T), _stream(pw.data.device)))
    return T


def quant_act(X: torch.Tensor, out=None):
    """bt_quant_act: per-token absmax int8. Returns (Xq [M, act_row_bytes(K)] int8, s_x [M], x_sum [M])."""
    _need(X, "X", torch.float32)
    M, K = X.shape
    dev = X.device
    if out is None:
        Xq = torch.empty((M, act_row_bytes(K)), dtype=torch.int8, device=dev)
        sx = torch.empty(M, dtype=torch.float32, device=dev)
        xsum = torch.empty(M, dtype=torch.int32, device=dev)
    else:
        Xq, sx, xsum = out
        _need(Xq, "Xq", torch.int8, (M, act_row_bytes(K)), dev)
        _need(sx, "s_x", torch.float32, (M,), dev)
        _need(xsum, "x_sum", torch.int32, (M,), dev)
    check(lib().bt_quant_act(_ptr(X), M, K, _ptr(Xq), _ptr(sx), _ptr(xsum), _stream(dev)))
    return Xq, sx, xsum


def _product(fn_name, pw: PackedWeight, q, want_y, want_acc, out_y, out_acc, algo=None, extra=()):
    pw.check()
    dev = pw.data.device
    M = _check_q(q, pw.K, dev)
    Xq, sx, xsum = q
    Y, acc = _outputs(M, pw.N, dev, want_y, want_acc, out_y, out_acc)
    args = [_ptr(pw.data), _ptr(pw.scale), _ptr(Xq), _ptr(sx), _ptr(xsum), M, pw.N, pw.K, _ptr(Y), _ptr(acc)]
    if algo is not None:
        args.append(algo)
    args.extend(extra)
    check(getattr(lib(), fn_name)(*args, _stream(dev)))
    return Y, acc


def ternary_gemv(pw: PackedWeight, q, want_y=True, want_acc=False, out_y=None, out_acc=None, algo=GEMV_AUTO):
    """bt_ternary_gemv_algo (bt_ternary_gemv_rs for row scales): decode product for M <= 16
    tokens. Returns (Y, acc)."""
    fn = "bt_ternary_gemv_rs" if pw.row_scales else "bt_ternary_gemv_algo"
    return _product(fn, pw, q, want_y, want_acc, out_y, out_acc, algo)


def gemm_workspace_bytes(M: int, N: int, K: int) -> int:
    """bt_gemm_workspace_bytes: workspace the split-K route of bt_ternary_gemm_ws uses (0: none)."""
    return int(lib().bt_gemm_workspace_bytes(M, N, K))


def gemm_split_plan(M: int, N: int, K: int) -> tuple[int, int]:
    """bt_gemm_split_plan: (full_tiles, splits) -- the first full_tiles 64 x 256 output tiles
    are computed whole, each later one over `splits` workgroups (splits == 1: no split)."""
    full = ctypes.c_int64(0)
    splits = ctypes.c_int32(0)
    check(lib().bt_gemm_split_plan(M, N, K, ctypes.byref(full), ctypes.byref(splits)))
    return int(full.value), int(splits.value)


def gemm_workspace(M: int, N: int, K: int, device) -> torch.Tensor | None:
    """A zero-filled workspace for bt_ternary_gemm_ws(M, N, K), or None when the shape does not split."""
    n = gemm_workspace_bytes(M, N, K)
    return torch.zeros(n, dtype=torch.uint8, device=device) if n else None


def ternary_gemm(pw: PackedWeight, q, want_y=True, want_acc=False, out_y=None, out_acc=None,
                 workspace: torch.Tensor | None = None):
    """bt_ternary_gemm: prefill product on int8 MFMA for any M. Returns (Y, acc).

    With a workspace (see gemm_workspace) the call is bt_ternary_gemm_ws, which splits K
    over several workgroups per tile where that pays; results are identical.
    """
    if workspace is None and not pw.row_scales:
        return _product("bt_ternary_gemm", pw, q, want_y, want_acc, out_y, out_acc)
    if workspace is not None:
        # any size is valid: one below gemm_workspace_bytes selects the unsplit route
        _need_bytes(workspace, "workspace", 0, pw.data.device)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return _product("bt_ternary_gemm_rs" if pw.row_scales else "bt_ternary_gemm_ws", pw, q, want_y, want_acc,
                    out_y, out_acc, extra=(_ptr(workspace), nbytes))


def linear_workspace_bytes(M: int, N: int, K: int) -> int:
    return int(lib().bt_linear_workspace_bytes(M, N, K))


def linear(X: torch.Tensor, pw: PackedWeight, want_y=True, want_acc=False, out_y=None, out_acc=None,
           workspace: torch.Tensor | None = None):
    """bt_ternary_linear: fp32 X [M,K] in, (Y [M,N] fp32, acc [M,N] int32) out.

    One fused launch for decode-sized M; quantize + GEMV/GEMM otherwise.
    """
    pw.check()
    dev = pw.data.device
    if X.dim() != 2:
        raise ValueError(f"X must be [M, K], got shape {tuple(X.shape)}")
    _need(X, "X", torch.float32, device=dev)
    M, K = X.shape
    if K != pw.K:
        raise ValueError(f"X has K = {K}, weights have K = {pw.K}")
    Y, acc = _outputs(M, pw.N, dev, want_y, want_acc, out_y, out_acc)
    ws_bytes = linear_workspace_bytes(M, pw.N, K)
    if ws_bytes and workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    elif ws_bytes:
        _need_bytes(workspace, "workspace", ws_bytes, dev)
    fn = lib().bt_ternary_linear_rs if pw.row_scales else lib().bt_ternary_linear
    check(fn(_ptr(pw.data), _ptr(pw.scale), _ptr(X), M, pw.N, K, _ptr(Y), _ptr(acc),
             _ptr(workspace) if ws_bytes else 0, _stream(dev)))
    return Y, acc


STATIC_SCRATCH_BYTES = 64 << 20  # BT_STATIC_SCRATCH_BYTES


def linear_static(X: torch.Tensor, pw: PackedWeight, out_y=None, out_acc=None, want_y=True, want_acc=False):
    """bt_ternary_linear_static: bt_ternary_linear without a workspace (the library's static
    scratch serves the routes that need one). One scale per matrix only. Pass out_y / out_acc
    to keep the call free of allocation."""
    if pw.row_scales:
        raise ValueError("bt_ternary_linear_static takes weights with one scale per matrix")
    pw.check()
    dev = pw.data.device
    if X.dim() != 2:
        raise ValueError(f"X must be [M, K], got shape {tuple(X.shape)}")
    _need(X, "X", torch.float32, device=dev)
    M, K = X.shape
    if K != pw.K:
        raise ValueError(f"X has K = {K}, weights have K = {pw.K}")
    Y, acc = _outputs(M, pw.N, dev, want_y, want_acc, out_y, out_acc)
    check(lib().bt_ternary_linear_static(_ptr(pw.data), _ptr(pw.scale), _ptr(X), M, pw.N, K, _ptr(Y), _ptr(acc),
                                         _stream(dev)))
    return Y, acc


CALL_LINEAR, CALL_GEMV, CALL_GEMM, CALL_GEMM_WS, CALL_QUANT = 0, 1, 2, 3, 4


def kernel_plan(call: int, M: int, N: int, K: int, algo: int = GEMV_AUTO, row_scales: bool = False) -> str:
    """bt_kernel_plan: the kernel instances the call would launch (host-only query)."""
    buf = ctypes.create_string_buffer(512)
    check(lib().bt_kernel_plan(call, M, N, K, algo, int(row_scales), buf, len(buf)))
    return buf.value.decode()


# ------------------------------------------------------------- 1-bit activations
BITS_PLAIN, BITS_CODES = 1, 2


def pack_weights_binary(W: torch.Tensor, workspace: torch.Tensor | None = None) -> PackedWeight:
    """bt_pack_weights_binary: sign bits of W [N,K] fp32 and its absmax (W1A1 weights)."""
    _need(W, "W", torch.float32)
    N, K = W.shape
    dev = W.device
    data = torch.empty(max(int(lib().bt_binary_weight_bytes(N, K)), 16), dtype=torch.uint8, device=dev)
    scale = torch.empty(1, dtype=torch.float32, device=dev)
    ws_bytes = pack_workspace_bytes(N, K)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 8), dtype=torch.uint8, device=dev)
    else:
        _need_bytes(workspace, "workspace", ws_bytes, dev)
    check(lib().bt_pack_weights_binary(_ptr(W), N, K, _ptr(data), _ptr(scale), _ptr(workspace), _stream(dev)))
    return PackedWeight(data, scale, N, K)


def binarize_act(X: torch.Tensor, layout: int, out=None):
    """bt_binarize_act: (bits [M, row_bytes / 4] int32, x_scale [M] = absmax per token)."""
    _need(X, "X", torch.float32)
    M, K = X.shape
    dev = X.device
    words = int(lib().bt_act_bits_row_bytes(K, layout)) // 4
    if out is None:
        Xb = torch.empty((M, words), dtype=torch.int32, device=dev)
        sx = torch.empty(M, dtype=torch.float32, device=dev)
    else:
        Xb, sx = out
        _need(Xb, "Xb", torch.int32, (M, words), dev)
        _need(sx, "x_scale", torch.float32, (M,), dev)
    check(lib().bt_binarize_act(_ptr(X), M, K, layout, _ptr(Xb), _ptr(sx), _stream(dev)))
    return Xb, sx


def _bits_product(fn_name, pw: PackedWeight, b, layout, want_y, want_acc, out_y, out_acc):
    dev = pw.data.device
    pw.check(int(lib().bt_binary_weight_bytes(pw.N, pw.K)) if layout == BITS_PLAIN else None)
    Xb, sx = b
    if not isinstance(sx, torch.Tensor) or sx.dim() != 1:
        raise ValueError("x_scale must be a 1-D tensor of M scales")
    M = sx.shape[0]
    _need(Xb, "Xb", torch.int32, (M, int(lib().bt_act_bits_row_bytes(pw.K, layout)) // 4), dev)
    _need(sx, "x_scale", torch.float32, (M,), dev)
    Y, acc = _outputs(M, pw.N, dev, want_y, want_acc, out_y, out_acc)
    check(getattr(lib(), fn_name)(_ptr(pw.data), _ptr(pw.scale), _ptr(Xb), _ptr(sx), M, pw.N, pw.K, _ptr(Y),
                                  _ptr(acc), _stream(dev)))
    return Y, acc


def binary_gemv(pw: PackedWeight, b, want_y=True, want_acc=False, out_y=None, out_acc=None):
    """bt_binary_gemv (W1A1): ``pw`` from pack_weights_binary, ``b`` from binarize_act(X, BITS_PLAIN)."""
    return _bits_product("bt_binary_gemv", pw, b, BITS_PLAIN, want_y, want_acc, out_y, out_acc)


def ternary_gemv_a1(pw: PackedWeight, b, want_y=True, want_acc=False, out_y=None, out_acc=None):
    """bt_ternary_gemv_a1 (W1.58A1): ``pw`` from pack_weights, ``b`` from binarize_act(X, BITS_CODES)."""
    return _bits_product("bt_ternary_gemv_a1", pw, b, BITS_CODES, want_y, want_acc, out_y, out_acc)
