"""Seeded synthetic inputs shaped like BitNet b1.58 linear layers.

This module draws random numbers and nothing else: it holds none of the method's
arithmetic (no scale, no rounding, no packing), so the CPU oracle and the HIP path
can both be fed from it without sharing any of the computation under test.

Recipe (the same everywhere):
  * NumPy ``default_rng(seed)`` (PCG64), ``standard_normal(dtype=float32)``;
  * activations X ~ N(0, 1); weights W = float32(0.02) * N(0, 1) in fp32;
  * the tiny matmul draws W [512,256] then X [128,256] from one generator, seed 0
    (shapes of the usage example on the "BitCompute" page, section "Usage");
  * layer weights use seed 1000*config + 10*layer + j and activations seed
    2000*config + j, with j = 0 QKV, 1 O, 2 gate+up, 3 down.

The layer shapes below are the 2B (BitNet-b1.58-2B-4T class: hidden 2560, FFN 6912),
7B (hidden 4096, FFN 11008, as in the "bit-floor" page's mem-estimate example) and
100B-class (hidden 8192, FFN 28672) linear layers, each as (N out, K in) with the fused
QKV and gate+up projections counted as one matrix.
"""
from __future__ import annotations

import numpy as np

WEIGHT_STD = np.float32(0.02)

# (name, N, K) per linear layer of one transformer block.
SHAPES_2B = (("qkv", 3840, 2560), ("o", 2560, 2560), ("gate_up", 13824, 2560), ("down", 2560, 6912))
SHAPES_7B = (("qkv", 12288, 4096), ("o", 4096, 4096), ("gate_up", 22016, 4096), ("down", 4096, 11008))
SHAPES_100B = (("qkv", 10240, 8192), ("o", 8192, 8192), ("gate_up", 57344, 8192), ("down", 8192, 28672))

# The 1-bit-activation GEMV shapes the bit-floor page benchmarks: (weight kind, N, K).
SHAPES_ONEBIT = (("binary", 4096, 4096), ("ternary", 4096, 4096), ("ternary", 11008, 4096))

# Workload ids used for seeding.
CFG_TINY, CFG_2B_DECODE, CFG_7B_DECODE, CFG_2B_PREFILL, CFG_100B_DECODE, CFG_ONEBIT = 1, 2, 3, 4, 5, 6

# Row groups of the fused matrices (the model's separate matrices stacked in output-row
# order): Q, K, V (grouped-query attention: K and V narrower at 2B and 100B) and gate, up.
# Every other matrix is one group.
_FUSED_GROUPS = {
    "2b": {"qkv": (2560, 640, 640), "gate_up": (6912, 6912)},
    "7b": {"qkv": (4096, 4096, 4096), "gate_up": (11008, 11008)},
    "100b": {"qkv": (8192, 1024, 1024), "gate_up": (28672, 28672)},
}
_CFG_MODEL = {CFG_2B_DECODE: "2b", CFG_2B_PREFILL: "2b", CFG_7B_DECODE: "7b", CFG_100B_DECODE: "100b"}


def row_groups(cfg: int, name: str, N: int) -> tuple:
    """Row counts of the groups of matrix ``name`` (N rows) in workload ``cfg``."""
    groups = _FUSED_GROUPS.get(_CFG_MODEL.get(cfg, ""), {}).get(name, (N,))
    assert sum(groups) == N, (cfg, name, N, groups)
    return groups


def gaussian(shape, seed: int, std=None) -> np.ndarray:
    """fp32 N(0,1) draws from PCG64(seed), optionally times a fp32 std."""
    z = np.random.default_rng(seed).standard_normal(shape, dtype=np.float32)
    if std is not None:
        z = np.float32(std) * z
    return np.ascontiguousarray(z, dtype=np.float32)


def weight_seed(config: int, layer: int, j: int) -> int:
    return 1000 * config + 10 * layer + j


def act_seed(config: int, j: int) -> int:
    return 2000 * config + j


def layer_weight(config: int, layer: int, j: int, N: int, K: int) -> np.ndarray:
    """W [N,K] fp32 = 0.02 * N(0,1) for weight matrix j of a layer."""
    return gaussian((N, K), weight_seed(config, layer, j), WEIGHT_STD)


def layer_activation(config: int, j: int, M: int, K: int) -> np.ndarray:
    """X [M,K] fp32 ~ N(0,1) feeding weight matrix j."""
    return gaussian((M, K), act_seed(config, j))


def tiny_matmul():
    """(W [512,256], X [128,256]) from one PCG64(0) stream, W drawn first."""
    rng = np.random.default_rng(0)
    W = WEIGHT_STD * rng.standard_normal((512, 256), dtype=np.float32)
    X = rng.standard_normal((128, 256), dtype=np.float32)
    return np.ascontiguousarray(W, np.float32), np.ascontiguousarray(X, np.float32)


def device_gaussian(shape, seed: int, device, std=None):
    """fp32 N(0,1) drawn directly on a torch device from a seeded torch.Generator.

    For resident weight sets too large to draw on the host (hundreds of MB packed,
    several GB as fp32). Different stream from ``gaussian``: use it only where no
    host-side copy of the same tensor is compared against.
    """
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed)
    z = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std is not None:
        z.mul_(float(np.float32(std)))
    return z
