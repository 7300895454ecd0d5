"""The whole-layer calls under HIP graph capture. Each route of bt_ternary_linear (the fused
decode kernel at eight and at two k-splits, quantizer + staged GEMV, quantizer + the small-M
GEMM, quantizer + GEMM with every tile split in K, quantizer + GEMM with the last round split)
and bt_ternary_linear_static is captured once and replayed with new inputs. Between replays
the program runs its own eager work on the same workspace and synchronizes; every replay must
give acc and Y bit-identical to an eager call on the same inputs (the split-K arrival
counters, which the quantizer launch zero-fills and the last split resets, must be back at
zero for every replay). The eager calls themselves are checked against the oracle by the
other parity modules; here the small cases are also checked against the oracle directly.
"""
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import oracle
import bit_ternary_weight_absmean_amd as bt
from bit_ternary_weight_absmean_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def note(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def same_bits(a: torch.Tensor, b: torch.Tensor) -> bool:
    x, y = a.cpu().numpy(), b.cpu().numpy()
    return x.shape == y.shape and np.array_equal(x.view(np.uint32), y.view(np.uint32))


# (M, N, K): fused S = 8, fused S = 2, quantizer + staged GEMV, quantizer + the small-M GEMM
# form (3-stage and 2-stage ring), quantizer + GEMM split in K (every tile), quantizer + GEMM
# with the last round's tiles split.
ROUTES = [(1, 3840, 2560), (4, 13824, 2560), (16, 2560, 2560), (256, 2560, 2560), (300, 3500, 2600),
          (650, 3300, 5500), (2048, 2560, 6912)]


@pytest.mark.parametrize("static", [False, True], ids=["workspace", "static"])
@pytest.mark.parametrize("M,N,K", ROUTES)
def test_linear_graph_replay(M, N, K, static):
    plan = bt.kernel_plan(bt.CALL_LINEAR, M, N, K)
    note(f"graph linear M={M} N={N} K={K} static={static} plan={plan}")
    W = synth.gaussian((N, K), 7300 + N + K, 0.02)
    pw = bt.pack_weights(torch.from_numpy(W).to(DEV))
    ws_bytes = bt.linear_workspace_bytes(M, N, K)
    ws = None if static or ws_bytes == 0 else torch.empty(ws_bytes, dtype=torch.uint8, device=DEV)
    xin = torch.zeros((M, K), dtype=torch.float32, device=DEV)
    Y = torch.empty((M, N), dtype=torch.float32, device=DEV)
    acc = torch.empty((M, N), dtype=torch.int32, device=DEV)

    def call(X, out_y, out_acc):
        if static:
            return bt.linear_static(X, pw, out_y=out_y, out_acc=out_acc)
        return bt.linear(X, pw, out_y=out_y, out_acc=out_acc, workspace=ws)

    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        call(xin, Y, acc)  # eager warm-up on the capture stream (and the scratch lookup)
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call(xin, Y, acc)
    other_y = torch.empty_like(Y)
    other_acc = torch.empty_like(acc)
    for rep in range(3):
        X = synth.gaussian((M, K), 7400 + 10 * rep + M)
        xin.copy_(torch.from_numpy(X).to(DEV))
        # the program's own eager work between replays, on the same workspace or scratch
        with torch.cuda.stream(s):
            call(torch.from_numpy(synth.gaussian((M, K), 7500 + rep)).to(DEV), other_y, other_acc)
        s.synchronize()
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            g.replay()
        s.synchronize()
        eager_y, eager_acc = bt.linear(xin, pw, want_acc=True)
        torch.cuda.synchronize()
        assert np.array_equal(acc.cpu().numpy(), eager_acc.cpu().numpy()), f"replay {rep}: acc"
        assert same_bits(Y, eager_y), f"replay {rep}: Y"
        if M * N * K <= 2e9:
            ref = oracle.linear(W, X)
            np.testing.assert_array_equal(acc.cpu().numpy(), ref["acc"])


_FIRST_STATIC_UNDER_CAPTURE = r"""
import sys
import numpy as np
import torch
sys.path.insert(0, {root!r})
import bit_ternary_weight_absmean_amd as bt
from bit_ternary_weight_absmean_amd import synth

M, N, K = 16, 2560, 2560  # a route that uses the static scratch
dev = "cuda:0"
pw = bt.pack_weights(torch.from_numpy(synth.gaussian((N, K), 7601, 0.02)).to(dev))
X = torch.from_numpy(synth.gaussian((M, K), 7602)).to(dev)
Y = torch.empty((M, N), dtype=torch.float32, device=dev)
acc = torch.empty((M, N), dtype=torch.int32, device=dev)
torch.cuda.synchronize()
s = torch.cuda.Stream()
g = torch.cuda.CUDAGraph()
with torch.cuda.graph(g, stream=s):
    bt.linear_static(X, pw, out_y=Y, out_acc=acc)  # the process's first static call
for rep in range(2):
    with torch.cuda.stream(s):
        g.replay()
    s.synchronize()
    ey, ea = bt.linear(X, pw, want_acc=True)
    torch.cuda.synchronize()
    assert np.array_equal(acc.cpu().numpy(), ea.cpu().numpy()), "acc"
    assert np.array_equal(Y.cpu().numpy().view(np.uint32), ey.cpu().numpy().view(np.uint32)), "Y"
print("first static call under capture: ok", flush=True)
"""


def test_first_static_call_under_capture():
    """A process whose first bt_ternary_linear_static call (the one that looks up the static
    scratch's device address) is made under graph capture: the capture and its replays work."""
    note("first static call under capture (child process)")
    run = subprocess.run([sys.executable, "-c", _FIRST_STATIC_UNDER_CAPTURE.format(root=ROOT)],
                         capture_output=True, text=True, timeout=240, cwd=ROOT)
    print(run.stdout[-2000:], run.stderr[-2000:])
    assert run.returncode == 0, run.stderr[-2000:]
    assert "ok" in run.stdout
