"""The C ABI from plain C. tests/c_abi/bt_c_client.c links libbt.so, the HIP runtime and the
C oracle, and runs pack, quantize, every product entry point and the whole-layer calls on six
shapes (the tiny matmul, 2B-class decode on the fused and the staged route, a ragged shape
with K % 4 != 0, prefill with split-K), plus argument errors, checking each result against
the oracle: codes, gamma, q, s_x, sum q and acc bit-exact, Y within 1e-5 |Y| + 1e-6.

CPU: the program builds with -Werror and links (every entry point it calls resolves in
libbt.so); without a GPU it exits 77 having run nothing. GPU: it runs every case and exits 0.
"""
import shutil
import subprocess

import pytest

from tests import c_abi

pytestmark = pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")


def _program() -> str:
    if c_abi.stale():
        c_abi.build()
    return c_abi.EXE


def test_c_client_builds_and_links():
    exe = _program()
    run = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    # no GPU: 77 and nothing run; a GPU that is visible here runs the whole program
    assert run.returncode in (0, 77), run.stdout + run.stderr
    if run.returncode == 77:
        assert "no GPU" in run.stdout


@pytest.mark.gpu
def test_c_client_matches_oracle():
    exe = _program()
    print(f"running {exe}", flush=True)
    run = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    print(run.stdout)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "all checks passed" in run.stdout
