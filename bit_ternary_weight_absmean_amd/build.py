"""Build libbt.so (HIP, gfx950 only) in-tree with hipcc.

    python -m bit_ternary_weight_absmean_amd.build

Each .hip source is compiled to an object in parallel, then linked into
``bit_ternary_weight_absmean_amd/libbt.so``; the benchmark's ceiling kernels go into
``libbt_ceilings.so`` beside it.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG, "_build")
LIB_PATH = os.path.join(PKG, "libbt.so")
# The benchmark's ceiling kernels (empty launch, plain read, MFMA loop): a library of their
# own, not part of libbt.so.
CEILINGS_SRC = "ceilings.hip"
CEILINGS_LIB = os.path.join(PKG, "libbt_ceilings.so")
ARCH = "gfx950"

SOURCES = ["abi.hip", "pack.hip", "quant.hip", "gemv.hip", "lut.hip", "bits.hip", "decode.hip", "gemm.hip"]

COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # IEEE fp32 behaviour the quantizer's bit-exactness relies on: no contraction,
    # denormals kept, correctly rounded fp32 division.
    "-ffp-contract=off",
    "-fno-gpu-flush-denormals-to-zero",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    # Keep the compiler from emitting packed fp32 VALU ops.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # Kernel arguments arrive preloaded in SGPRs (gfx950): a decode launch does not wait
    # on a kernarg memory load before it can form its first addresses.
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
    "-Wno-unused-command-line-argument",
    "-I", INCLUDE,
    "-I", CSRC,
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the HIP library cannot be built")
    return path


# Per-source extra flags. The MFMA-loop ceiling keeps its sixteen accumulators in VGPRs:
# with AGPR accumulators the compiler copies them between AGPRs inside the loop.
EXTRA_FLAGS = {CEILINGS_SRC: ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *COMMON_FLAGS, *EXTRA_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every HIP source for gfx950 and link libbt.so; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), 8)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB_PATH)
    obj = _compile(CEILINGS_SRC)
    tmp = CEILINGS_LIB + ".tmp"
    res = subprocess.run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, obj], capture_output=True,
                         text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, CEILINGS_LIB)
    if verbose:
        print(f"built {LIB_PATH} and {CEILINGS_LIB}")
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
