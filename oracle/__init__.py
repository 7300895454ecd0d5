"""CPU oracle for the BitNet b1.58 W1.58A8 ternary linear layer (test infrastructure).

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py``
import this package. The product path (``bit_ternary_weight_absmean_amd``) never
imports it and shares no code with it.

The arithmetic lives in ``bt_oracle.c`` (plain C, fp64 where the method leaves the
precision open); this module only compiles it with gcc and marshals NumPy arrays.
Each wrapper cites the page passage that its C function follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "bt_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
# -fno-fast-math / -ffp-contract=off: every float operation is the one IEEE op the
# source names; no FMA contraction, no reassociation, no flush-to-zero.
CFLAGS = ["-O2", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared", "-std=c11"]

_lib = None


class OracleInputError(ValueError):
    """Raised when an input lies outside the contract (non-finite values)."""


def build(out_path: str = _LIB_PATH, src: str = _SRC) -> str:
    """Compile the oracle with gcc into a shared library and return its path."""
    cmd = ["gcc", *CFLAGS, "-o", out_path, src, "-lm"]
    subprocess.run(cmd, check=True)
    return out_path


def _bind(lib: ctypes.CDLL) -> ctypes.CDLL:
    i64, vp = ctypes.c_int64, ctypes.c_void_p
    lib.oracle_absmean.argtypes = [vp, i64, i64, vp]
    lib.oracle_ternarize.argtypes = [vp, i64, i64, ctypes.c_float, vp]
    lib.oracle_quant_act.argtypes = [vp, i64, i64, vp, vp, vp]
    lib.oracle_ternary_matmul.argtypes = [vp, vp, i64, i64, i64, vp]
    lib.oracle_scale_epilogue.argtypes = [vp, ctypes.c_float, vp, i64, i64, vp]
    lib.oracle_absmean_rows.argtypes = [vp, i64, i64, vp, i64, vp]
    lib.oracle_ternarize_rows.argtypes = [vp, i64, i64, vp, vp]
    lib.oracle_scale_epilogue_rows.argtypes = [vp, vp, vp, i64, i64, vp]
    lib.oracle_absmax_rows.argtypes = [vp, i64, i64, vp]
    lib.oracle_binarize.argtypes = [vp, i64, i64, vp]
    for f in ("oracle_absmean", "oracle_ternarize", "oracle_quant_act",
              "oracle_ternary_matmul", "oracle_scale_epilogue", "oracle_absmean_rows",
              "oracle_ternarize_rows", "oracle_scale_epilogue_rows", "oracle_absmax_rows",
              "oracle_binarize"):
        getattr(lib, f).restype = ctypes.c_int
    return lib


def load(path: str | None = None) -> ctypes.CDLL:
    """Load the compiled oracle, building it first only if no library exists."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        _lib = _bind(ctypes.CDLL(_LIB_PATH))
    return _lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _f32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32)


def _check(rc: int) -> None:
    if rc == 2:
        raise OracleInputError("the row groups do not cover the rows exactly")
    if rc != 0:
        raise OracleInputError("oracle rejected a non-finite input")


def absmean(W, lib=None) -> np.float32:
    """gamma = mean|W| (fp64 two-level sum, one rounding to fp32).

    "bit-floor" page, "What's inside" (pack.rs: mean-abs scale for ternary weights).
    """
    lib = lib or load()
    W = _f32(W)
    N, K = W.shape
    out = np.zeros(1, dtype=np.float32)
    _check(lib.oracle_absmean(_ptr(W), N, K, _ptr(out)))
    return out[0]


def ternarize(W, gamma, lib=None) -> np.ndarray:
    """t = RoundClip(W/gamma, -1, 1) as int8, via the exact compare |w| > gamma/2.

    "bit-floor" page, "What's inside" (pack.rs: mean-abs threshold zero-suppression).
    """
    lib = lib or load()
    W = _f32(W)
    N, K = W.shape
    T = np.empty((N, K), dtype=np.int8)
    _check(lib.oracle_ternarize(_ptr(W), N, K, ctypes.c_float(float(gamma)), _ptr(T)))
    return T


def quant_act(X, lib=None):
    """Per-token absmax int8: returns (Q int8 [M,K], s_x fp32 [M], qsum int32 [M]).

    BitNet GPU guide, "Understanding the Two-Phase Architecture"; "bit-floor" page,
    "What's inside" (scale.rs).
    """
    lib = lib or load()
    X = _f32(X)
    M, K = X.shape
    Q = np.empty((M, K), dtype=np.int8)
    s = np.empty(M, dtype=np.float32)
    qs = np.empty(M, dtype=np.int32)
    _check(lib.oracle_quant_act(_ptr(X), M, K, _ptr(Q), _ptr(s), _ptr(qs)))
    return Q, s, qs


def ternary_matmul(T, Q, lib=None) -> np.ndarray:
    """acc[m,n] = sum_k T[n,k] * Q[m,k] (int32 naive triple loop).

    "BitCompute" page, "Features"; "bit-floor" page, "The core math".
    """
    lib = lib or load()
    T = np.ascontiguousarray(T, dtype=np.int8)
    Q = np.ascontiguousarray(Q, dtype=np.int8)
    N, K = T.shape
    M, K2 = Q.shape
    if K != K2:
        raise ValueError(f"K mismatch: T has {K}, Q has {K2}")
    acc = np.empty((M, N), dtype=np.int32)
    _check(lib.oracle_ternary_matmul(_ptr(T), _ptr(Q), M, N, K, _ptr(acc)))
    return acc


def scale_epilogue(acc, gamma, s_x, lib=None) -> np.ndarray:
    """y = acc * gamma * s_x[m] in fp64, rounded once to fp32.

    "bit-floor" page, "The core math" (scale_w x scale_x x integer dot).
    """
    lib = lib or load()
    acc = np.ascontiguousarray(acc, dtype=np.int32)
    s_x = _f32(s_x)
    M, N = acc.shape
    Y = np.empty((M, N), dtype=np.float32)
    _check(lib.oracle_scale_epilogue(_ptr(acc), ctypes.c_float(float(gamma)), _ptr(s_x),
                                     M, N, _ptr(Y)))
    return Y


def linear(W, X, lib=None) -> dict:
    """The whole W1.58A8 linear layer: every intermediate of the path, as a dict."""
    lib = lib or load()
    gamma = absmean(W, lib)
    T = ternarize(W, gamma, lib)
    Q, s_x, qsum = quant_act(X, lib)
    acc = ternary_matmul(T, Q, lib)
    Y = scale_epilogue(acc, gamma, s_x, lib)
    return {"gamma": gamma, "T": T, "Q": Q, "s_x": s_x, "qsum": qsum, "acc": acc, "Y": Y}


def absmean_rows(W, seg_rows=None, lib=None) -> np.ndarray:
    """Row-group scales: row_scale[n] = mean|W| over row n's group (fp32 [N]).

    ``seg_rows`` lists the group sizes in row order (None: one group per row).
    BitNet GPU guide, "Frequently Asked Questions" (model-specific scales and group
    dimensions).
    """
    lib = lib or load()
    W = _f32(W)
    N, K = W.shape
    out = np.empty(N, dtype=np.float32)
    if seg_rows is None:
        _check(lib.oracle_absmean_rows(_ptr(W), N, K, None, 0, _ptr(out)))
    else:
        seg = np.ascontiguousarray(seg_rows, dtype=np.int64)
        _check(lib.oracle_absmean_rows(_ptr(W), N, K, _ptr(seg), len(seg), _ptr(out)))
    return out


def ternarize_rows(W, row_scale, lib=None) -> np.ndarray:
    """Codes of each row against its own scale (the exact compare of ``ternarize``)."""
    lib = lib or load()
    W = _f32(W)
    N, K = W.shape
    rs = _f32(row_scale)
    T = np.empty((N, K), dtype=np.int8)
    _check(lib.oracle_ternarize_rows(_ptr(W), N, K, _ptr(rs), _ptr(T)))
    return T


def scale_epilogue_rows(acc, row_scale, s_x, lib=None) -> np.ndarray:
    """y = acc * gamma_n * s_x[m] in fp64, rounded once to fp32.

    "bit-floor" page, "The core math", with the weight scale of output row n.
    """
    lib = lib or load()
    acc = np.ascontiguousarray(acc, dtype=np.int32)
    rs, s_x = _f32(row_scale), _f32(s_x)
    M, N = acc.shape
    Y = np.empty((M, N), dtype=np.float32)
    _check(lib.oracle_scale_epilogue_rows(_ptr(acc), _ptr(rs), _ptr(s_x), M, N, _ptr(Y)))
    return Y


def linear_rows(W, X, seg_rows=None, lib=None) -> dict:
    """The linear layer with row-group weight scales: every intermediate, as a dict."""
    lib = lib or load()
    row_scale = absmean_rows(W, seg_rows, lib)
    T = ternarize_rows(W, row_scale, lib)
    Q, s_x, qsum = quant_act(X, lib)
    acc = ternary_matmul(T, Q, lib)
    Y = scale_epilogue_rows(acc, row_scale, s_x, lib)
    return {"row_scale": row_scale, "T": T, "Q": Q, "s_x": s_x, "qsum": qsum, "acc": acc, "Y": Y}


def absmax_rows(V, lib=None) -> np.ndarray:
    """max |V[r, :]| per row (fp32 [R]); a matrix's absmax is absmax_rows(V.reshape(1, -1)).

    "bit-floor" page, "What's inside" (pack.rs / scale.rs: absmax scales).
    """
    lib = lib or load()
    V = _f32(V)
    R, C = V.shape
    out = np.empty(R, dtype=np.float32)
    _check(lib.oracle_absmax_rows(_ptr(V), R, C, _ptr(out)))
    return out


def binarize(V, lib=None) -> np.ndarray:
    """+1 where V >= 0, -1 elsewhere (int8), the 1-bit operands of "The core math"."""
    lib = lib or load()
    V = _f32(V)
    R, C = V.shape
    B = np.empty((R, C), dtype=np.int8)
    _check(lib.oracle_binarize(_ptr(V), R, C, _ptr(B)))
    return B


def binary_layer(W, X, lib=None) -> dict:
    """W1A1: y = max|W| * max|x_m| * sum_k sign(W) sign(x) ("bit-floor" page, "The core math")."""
    lib = lib or load()
    s_w = absmax_rows(np.asarray(W, np.float32).reshape(1, -1), lib)[0]
    Wb = binarize(W, lib)
    Xb = binarize(X, lib)
    s_x = absmax_rows(X, lib)
    acc = ternary_matmul(Wb, Xb, lib)
    Y = scale_epilogue(acc, s_w, s_x, lib)
    return {"s_w": s_w, "Wb": Wb, "Xb": Xb, "s_x": s_x, "acc": acc, "Y": Y}


def ternary_a1_layer(W, X, lib=None) -> dict:
    """W1.58A1: ternary weights (absmean, as in ``linear``) against binarized tokens."""
    lib = lib or load()
    gamma = absmean(W, lib)
    T = ternarize(W, gamma, lib)
    Xb = binarize(X, lib)
    s_x = absmax_rows(X, lib)
    acc = ternary_matmul(T, Xb, lib)
    Y = scale_epilogue(acc, gamma, s_x, lib)
    return {"gamma": gamma, "T": T, "Xb": Xb, "s_x": s_x, "acc": acc, "Y": Y}
