"""The C-ABI client test program: builds tests/c_abi/bt_c_client.c with gcc against
include/bt.h, the HIP runtime and the C oracle (oracle/bt_oracle.c), linked to the in-tree
libbt.so. Test infrastructure: run by tests/test_c_client.py."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "bt_c_client.c")
ORACLE_SRC = os.path.join(ROOT, "oracle", "bt_oracle.c")
PKG = os.path.join(ROOT, "bit_ternary_weight_absmean_amd")
LIB = os.path.join(PKG, "libbt.so")
EXE = os.path.join(HERE, "bt_c_client")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def command(out: str = EXE) -> list:
    # The library and the runtime are found through $ORIGIN-relative and ROCm rpaths, so the
    # program runs from a copy of the tree at any path.
    return ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
            "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"),
            SRC, ORACLE_SRC, "-o", out,
            "-L", PKG, "-lbt", "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-lm",
            "-Wl,-rpath,$ORIGIN/../../bit_ternary_weight_absmean_amd", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}"]


def stale() -> bool:
    """True when the program is missing or older than a source it is built from."""
    if not os.path.exists(EXE):
        return True
    t = os.path.getmtime(EXE)
    return any(os.path.getmtime(p) > t for p in (SRC, ORACLE_SRC, os.path.join(ROOT, "include", "bt.h"), LIB))


def build() -> str:
    """Compile and link the client; returns its path."""
    if not os.path.exists(LIB):
        raise RuntimeError(f"{LIB} is not built")
    res = subprocess.run(command(), capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"building the C client failed:\n{res.stdout}\n{res.stderr}")
    return EXE
