"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bar: gamma, ternary codes, int8 activations, s_x, sum q and the int32 accumulator
bit-exact; Y within |dY| <= 1e-5 |Y| + 1e-6. Inputs come from the seeded generators
in ``bit_ternary_weight_absmean_amd.synth``; expected values only from ``oracle``.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import bit_ternary_weight_absmean_amd as bt
from bit_ternary_weight_absmean_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def note(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def tol_ok(y, ref):
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    return bool(np.all(np.abs(y - ref) <= 1e-5 * np.abs(ref) + 1e-6))


def f32_bits(x):
    return np.asarray(x, np.float32).view(np.uint32)


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def gpu_pack(W):
    pw = bt.pack_weights(to_dev(W))
    return pw


def gpu_quant(X):
    return bt.quant_act(to_dev(X))


def oracle_layer(W, X):
    return oracle.linear(W, X)


def check_product(pw, q, ref, M, N, fn, **kw):
    Y, acc = fn(pw, q, want_y=True, want_acc=True, **kw)
    torch.cuda.synchronize()
    acc = acc.cpu().numpy()
    Y = Y.cpu().numpy()
    assert acc.shape == (M, N)
    bad = np.argwhere(acc != ref["acc"])
    assert bad.size == 0, f"{len(bad)} acc mismatches, first at {bad[:5].tolist()}"
    assert tol_ok(Y, ref["Y"])


# ------------------------------------------------------------------- pack
PACK_SHAPES = [(1, 1), (3, 7), (64, 64), (100, 300), (512, 256), (65, 129), (2560, 2560), (3840, 2560)]


@pytest.mark.parametrize("N,K", PACK_SHAPES)
def test_pack_gamma_and_codes(N, K):
    note(f"pack N={N} K={K}")
    W = synth.gaussian((N, K), 7000 + N + K, 0.02)
    pw = gpu_pack(W)
    T = bt.unpack_weights(pw)
    torch.cuda.synchronize()
    g_ref = oracle.absmean(W)
    assert f32_bits(pw.scale.cpu().numpy()[0]) == f32_bits(g_ref)
    np.testing.assert_array_equal(T.cpu().numpy(), oracle.ternarize(W, g_ref))


def test_pack_ties_and_padding():
    """Weights exactly at +-gamma/2 pack to 0; padded rows/columns are never visible."""
    note("pack ties")
    W = np.array([[0.75, -0.25, 0.25, 0.75]], np.float32)
    pw = gpu_pack(W)
    np.testing.assert_array_equal(bt.unpack_weights(pw).cpu().numpy(), [[1, 0, 0, 1]])
    assert pw.scale.item() == 0.5
    raw = pw.data.cpu().numpy().view(np.uint32)
    # chunk 0, row 0: word 0 holds codes k=0..15 -> codes 2,1,1,2 then padding code 1
    assert raw.size == 64 * 64 // 16
    assert np.all(raw[4:] == 0x55555555)  # rows 1..63 are all padding


def test_pack_zero_matrix():
    note("pack zero")
    W = np.zeros((70, 90), np.float32)
    pw = gpu_pack(W)
    assert pw.scale.item() == 0.0
    assert not bt.unpack_weights(pw).cpu().numpy().any()


# ------------------------------------------------------------------ quant
QUANT_SHAPES = [(1, 1), (1, 7), (3, 300), (1, 4), (2, 1028), (128, 256), (1, 2560), (1, 28672), (5, 6912),
                (2048, 2560), (3, 32768), (2, 40000), (3, 11008), (2, 20000), (4, 5120)]


@pytest.mark.parametrize("M,K", QUANT_SHAPES)
def test_quant_act(M, K):
    note(f"quant M={M} K={K}")
    X = synth.gaussian((M, K), 8000 + M + K)
    if M >= 3:
        X[1] = 0.0  # an all-zero token
    Xq, sx, xsum = gpu_quant(X)
    torch.cuda.synchronize()
    Q, s_ref, qs_ref = oracle.quant_act(X)
    Xq = Xq.cpu().numpy()
    assert Xq.shape == (M, bt.act_row_bytes(K))
    np.testing.assert_array_equal(Xq[:, :K], Q)
    assert not Xq[:, K:].any()
    np.testing.assert_array_equal(f32_bits(sx.cpu().numpy()), f32_bits(s_ref))
    np.testing.assert_array_equal(xsum.cpu().numpy(), qs_ref)


def test_quant_hand_ties():
    note("quant ties")
    X = np.array([[127.0, 62.5, -0.5, 1.5], [127.0, -1.5, -2.5, 3.5], [1.0, -2.0, 0.5, 0.25]], np.float32)
    Xq, sx, xsum = gpu_quant(X)
    np.testing.assert_array_equal(Xq.cpu().numpy()[:, :4], [[127, 62, 0, 2], [127, -2, -2, 4], [64, -127, 32, 16]])
    np.testing.assert_array_equal(xsum.cpu().numpy(), [191, 127, -15])


def test_quant_unaligned_rows():
    """K not a multiple of 4 and an input at a 4-byte (not 16-byte) offset."""
    note("quant unaligned")
    X = synth.gaussian((4, 4 * 133 + 1), 8100)
    big = torch.zeros(X.size + 1, dtype=torch.float32, device=DEV)
    big[1:] = to_dev(X.ravel())
    Xd = big[1:].view(4, -1)
    Xq, sx, xsum = bt.quant_act(Xd)
    Q, s_ref, qs_ref = oracle.quant_act(X)
    np.testing.assert_array_equal(Xq.cpu().numpy()[:, :X.shape[1]], Q)
    np.testing.assert_array_equal(xsum.cpu().numpy(), qs_ref)


# -------------------------------------------------------------- products
SMALL = [(1, 1, 1), (1, 100, 300), (2, 130, 129), (3, 65, 1000), (4, 512, 256), (5, 200, 700),
         (8, 64, 64), (16, 300, 517), (16, 1000, 2560)]


@pytest.mark.parametrize("M,N,K", SMALL)
@pytest.mark.parametrize("algo", [bt.GEMV_DOT4, bt.GEMV_MFMA, bt.GEMV_AUTO])
def test_gemv_small(M, N, K, algo):
    if algo == bt.GEMV_DOT4 and M > 4:
        pytest.skip("dot4 takes M <= 4")
    note(f"gemv algo={algo} M={M} N={N} K={K}")
    W = synth.gaussian((N, K), 9000 + N, 0.02)
    X = synth.gaussian((M, K), 9500 + M)
    ref = oracle_layer(W, X)
    check_product(gpu_pack(W), gpu_quant(X), ref, M, N, bt.ternary_gemv, algo=algo)


# (257, 516, 700): ragged 64 x 256 tiles in both dimensions with both outputs;
# (1024, 8448, 512): 528 tiles, more than one round of workgroups. K >= 512 with at most
# 256 tiles of 64 x 64 takes the small-M form (k_gemm_ks): (300, 200, 517), (64, 1000, 2560),
# (257, 516, 700), and its k-share edges: 4 steps (one per wave), 5 steps of 9 chunks
# (shares 2, 2, 1, 0), 5 whole steps, exactly 256 tiles (3-stage ring, one workgroup per CU)
# and 257 to 512 tiles (2-stage ring, two per CU; ragged, and exactly 512); and the longest
# rows (K = 28672: 112 steps, 28 per wave). The small-M form stores 16-byte row pieces where
# N % 4 == 0 and 4-byte fragments otherwise: (100, 130, 640) and (257, 515, 700) take the
# latter on the 3-stage ring, (300, 3501, 900) on the 2-stage one (275 tiles).
GEMM_SMALL = [(1, 64, 64), (17, 100, 300), (128, 512, 256), (129, 130, 129), (300, 200, 517), (64, 1000, 2560),
              (257, 516, 700), (1024, 8448, 512), (64, 64, 512), (200, 700, 513), (100, 130, 640),
              (256, 4096, 1024), (300, 3500, 900), (512, 4096, 768), (40, 1000, 28672), (257, 515, 700),
              (300, 3501, 900)]


@pytest.mark.parametrize("M,N,K", GEMM_SMALL)
def test_gemm_small(M, N, K):
    note(f"gemm M={M} N={N} K={K}")
    W = synth.gaussian((N, K), 9100 + N, 0.02)
    X = synth.gaussian((M, K), 9600 + M)
    ref = oracle_layer(W, X)
    check_product(gpu_pack(W), gpu_quant(X), ref, M, N, bt.ternary_gemm)


@pytest.mark.parametrize("M,N,K", [(300, 200, 517), (300, 3500, 900), (1024, 8448, 512)])
@pytest.mark.parametrize("shift_y,shift_acc", [(1, 0), (0, 3), (2, 2)])
def test_gemm_outputs_not_16_byte_aligned(M, N, K, shift_y, shift_acc):
    """Caller outputs that start 4, 8 or 12 bytes past a 16-byte boundary (views into larger
    buffers): both GEMM forms fall back to element stores there; the results match the oracle
    and no element outside the views is written."""
    note(f"gemm unaligned outputs M={M} N={N} K={K} shifts {shift_y} {shift_acc}")
    W = synth.gaussian((N, K), 9100 + N, 0.02)
    X = synth.gaussian((M, K), 9600 + M)
    ref = oracle_layer(W, X)
    ybuf = torch.full((M * N + 8,), 1234.5, dtype=torch.float32, device=DEV)
    abuf = torch.full((M * N + 8,), -7, dtype=torch.int32, device=DEV)
    Yv = ybuf[shift_y:shift_y + M * N].view(M, N)
    Av = abuf[shift_acc:shift_acc + M * N].view(M, N)
    assert (Yv.data_ptr() % 16 != 0) or (Av.data_ptr() % 16 != 0)
    bt.ternary_gemm(gpu_pack(W), gpu_quant(X), out_y=Yv, out_acc=Av)
    torch.cuda.synchronize()
    bad = np.argwhere(Av.cpu().numpy() != ref["acc"])
    assert bad.size == 0, f"{len(bad)} acc mismatches, first at {bad[:5].tolist()}"
    assert tol_ok(Yv.cpu().numpy(), ref["Y"])
    yb, ab = ybuf.cpu().numpy(), abuf.cpu().numpy()
    assert (yb[:shift_y] == 1234.5).all() and (yb[shift_y + M * N:] == 1234.5).all()
    assert (ab[:shift_acc] == -7).all() and (ab[shift_acc + M * N:] == -7).all()


def test_tiny_workload_all_paths():
    """The tiny matmul workload (X [128,256], W [512,256], seed 0): gemm at M=128, gemv per token."""
    note("tiny workload")
    W, X = synth.tiny_matmul()
    ref = oracle_layer(W, X)
    pw, q = gpu_pack(W), gpu_quant(X)
    check_product(pw, q, ref, 128, 512, bt.ternary_gemm)
    for m0 in (0, 16, 112):
        sub = {"acc": ref["acc"][m0:m0 + 16], "Y": ref["Y"][m0:m0 + 16]}
        qs = (q[0][m0:m0 + 16], q[1][m0:m0 + 16], q[2][m0:m0 + 16])
        check_product(pw, qs, sub, 16, 512, bt.ternary_gemv, algo=bt.GEMV_MFMA)
    for m0 in (0, 77, 127):
        sub = {"acc": ref["acc"][m0:m0 + 1], "Y": ref["Y"][m0:m0 + 1]}
        qs = (q[0][m0:m0 + 1], q[1][m0:m0 + 1], q[2][m0:m0 + 1])
        check_product(pw, qs, sub, 1, 512, bt.ternary_gemv, algo=bt.GEMV_DOT4)


# --------------------------------------------- full-size layer shapes
@pytest.mark.parametrize("j,name,N,K", [(j, *s) for j, s in enumerate(synth.SHAPES_2B)])
def test_2b_decode_shapes_full(j, name, N, K):
    """2B decode layer shapes at M=1 (every output compared), in the launch the benchmark uses."""
    note(f"2B {name} N={N} K={K}")
    W = synth.layer_weight(synth.CFG_2B_DECODE, 0, j, N, K)
    X = synth.layer_activation(synth.CFG_2B_DECODE, j, 1, K)
    ref = oracle_layer(W, X)
    pw, q = gpu_pack(W), gpu_quant(X)
    assert f32_bits(pw.scale.cpu().numpy()[0]) == f32_bits(ref["gamma"])
    for algo in (bt.GEMV_AUTO, bt.GEMV_DOT4, bt.GEMV_MFMA):
        check_product(pw, q, ref, 1, N, bt.ternary_gemv, algo=algo)
    # 2B prefill at M=256 on the same weight (gemm)
    X2 = synth.layer_activation(synth.CFG_2B_PREFILL, j, 256, K)
    q2 = gpu_quant(X2)
    Q2, s2, qs2 = oracle.quant_act(X2)
    T = oracle.ternarize(W, ref["gamma"])
    rows = np.arange(0, 256, 7)
    acc_ref = oracle.ternary_matmul(T, Q2[rows])
    Y2, acc2 = bt.ternary_gemm(pw, q2, want_acc=True)
    acc2 = acc2.cpu().numpy()
    np.testing.assert_array_equal(acc2[rows], acc_ref)
    assert tol_ok(Y2.cpu().numpy()[rows], oracle.scale_epilogue(acc_ref, ref["gamma"], s2[rows]))


@pytest.mark.parametrize("M", [1, 4, 8])
def test_7b_gate_up_decode(M):
    note(f"7B gate_up M={M}")
    j = 2
    name, N, K = synth.SHAPES_7B[j]
    W = synth.layer_weight(synth.CFG_7B_DECODE, 0, j, N, K)
    X = synth.layer_activation(synth.CFG_7B_DECODE, j, M, K)
    g = oracle.absmean(W)
    T = oracle.ternarize(W, g)
    assert abs(float(np.mean(T == 0)) - 0.3101) < 0.005  # "~1/3 zeros"
    Q, s, qs = oracle.quant_act(X)
    rows = np.arange(0, N, 5)
    acc_ref = oracle.ternary_matmul(T[rows], Q)
    pw, q = gpu_pack(W), gpu_quant(X)
    for algo in ((bt.GEMV_AUTO, bt.GEMV_DOT4, bt.GEMV_MFMA) if M <= 4 else (bt.GEMV_AUTO, bt.GEMV_MFMA)):
        Y, acc = bt.ternary_gemv(pw, q, want_acc=True, algo=algo)
        np.testing.assert_array_equal(acc.cpu().numpy()[:, rows], acc_ref)
        assert tol_ok(Y.cpu().numpy()[:, rows], oracle.scale_epilogue(acc_ref, g, s))


def test_100b_down_decode_m16():
    """The longest K (28672) at M = 16 on a 100B-class down projection, sampled rows."""
    note("100B down M=16")
    j, N, K = 3, 8192, 28672
    W = synth.layer_weight(synth.CFG_100B_DECODE, 0, j, N, K)
    X = synth.layer_activation(synth.CFG_100B_DECODE, j, 16, K)
    g = oracle.absmean(W)
    rows = np.arange(3, N, 11)
    T = oracle.ternarize(W[rows], g)
    Q, s, qs = oracle.quant_act(X)
    acc_ref = oracle.ternary_matmul(T, Q)
    pw, q = gpu_pack(W), gpu_quant(X)
    assert f32_bits(pw.scale.cpu().numpy()[0]) == f32_bits(g)
    for M, algo in ((16, bt.GEMV_MFMA), (1, bt.GEMV_DOT4), (1, bt.GEMV_MFMA)):
        qm = (q[0][:M], q[1][:M], q[2][:M])
        Y, acc = bt.ternary_gemv(pw, qm, want_acc=True, algo=algo)
        np.testing.assert_array_equal(acc.cpu().numpy()[:, rows], acc_ref[:M])


# Split-K route (bt_ternary_gemm_ws): shapes chosen so that the split heuristic picks
# 4, 3 and 2 workgroups for every tile, ragged in M, N and K (more than 512 tiles of
# 64 x 64, so the small-M form does not take them).
SPLIT_SHAPES = [(600, 3500, 6900, 4), (650, 3300, 5500, 3), (700, 3000, 4000, 2)]


def split_of(M, N, K):
    """Workgroups per split tile the library picks (1: no split)."""
    return bt.gemm_split_plan(M, N, K)[1]


def counters_zero(ws, M, N, K):
    """The arrival counters of the split tiles (the workspace's leading words) are zero."""
    full, splits = bt.gemm_split_plan(M, N, K)
    if splits == 1:
        return ws is None  # no split: no workspace either
    tiles = -(-M // 64) * -(-N // 256)
    return bool((ws[: 4 * (tiles - full)].view(torch.int32) == 0).all())


def sampled_rows(M, step=29):
    """Token rows in every 64-token tile row, the last row included."""
    return np.concatenate([np.arange(3, M, step), [M - 1]])


@pytest.mark.parametrize("M,N,K,S", SPLIT_SHAPES)
def test_gemm_split_k(M, N, K, S):
    note(f"gemm split-K M={M} N={N} K={K} S={S}")
    assert bt.gemm_split_plan(M, N, K) == (0, S)
    W = synth.gaussian((N, K), 9150 + N, 0.02)
    X = synth.gaussian((M, K), 9650 + M)
    g = oracle.absmean(W)
    T = oracle.ternarize(W, g)
    Q, s, qs = oracle.quant_act(X)
    rows = sampled_rows(M)
    acc_ref = oracle.ternary_matmul(T, Q[rows])
    pw, q = gpu_pack(W), gpu_quant(X)
    ws = bt.gemm_workspace(M, N, K, DEV)
    for _ in range(2):  # the second call relies on the first leaving the counters at zero
        Y, acc = bt.ternary_gemm(pw, q, want_acc=True, workspace=ws)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(acc.cpu().numpy()[rows], acc_ref)
        assert tol_ok(Y.cpu().numpy()[rows], oracle.scale_epilogue(acc_ref, g, s[rows]))
        assert counters_zero(ws, M, N, K)
    # bit-identical to the unsplit route
    Y1, a1 = bt.ternary_gemm(pw, q, want_acc=True)
    Y2, a2 = bt.ternary_gemm(pw, q, want_acc=True, workspace=ws)
    np.testing.assert_array_equal(a1.cpu().numpy(), a2.cpu().numpy())
    np.testing.assert_array_equal(f32_bits(Y1.cpu().numpy()), f32_bits(Y2.cpu().numpy()))


# Tail split: whole tiles for full rounds of one tile per CU, the last partial round's
# tiles split (ragged in M, N and K): 288 tiles -> 256 whole + 32 in 4; 356 tiles ->
# 256 whole + 100 in 2.
TAIL_SHAPES = [(1100, 4096, 6200, 256, 4), (250, 22700, 3100, 256, 2)]


@pytest.mark.parametrize("M,N,K,full,S", TAIL_SHAPES)
def test_gemm_tail_split(M, N, K, full, S):
    note(f"gemm tail split M={M} N={N} K={K}")
    assert bt.gemm_split_plan(M, N, K) == (full, S)
    W = synth.gaussian((N, K), 9160 + N, 0.02)
    X = synth.gaussian((M, K), 9660 + M)
    g = oracle.absmean(W)
    T = oracle.ternarize(W, g)
    Q, s, qs = oracle.quant_act(X)
    # sampled token rows in every 64-token tile row, the last one included
    rows = np.concatenate([np.arange(5, M, 61), [M - 1]])
    acc_ref = oracle.ternary_matmul(T, Q[rows])
    pw, q = gpu_pack(W), gpu_quant(X)
    ws = bt.gemm_workspace(M, N, K, DEV)
    for _ in range(2):  # the second call relies on the first leaving the counters at zero
        Y, acc = bt.ternary_gemm(pw, q, want_acc=True, workspace=ws)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(acc.cpu().numpy()[rows], acc_ref)
        assert tol_ok(Y.cpu().numpy()[rows], oracle.scale_epilogue(acc_ref, g, s[rows]))
        assert counters_zero(ws, M, N, K)
    Y1, a1 = bt.ternary_gemm(pw, q, want_acc=True)
    np.testing.assert_array_equal(a1.cpu().numpy(), acc.cpu().numpy())
    np.testing.assert_array_equal(f32_bits(Y1.cpu().numpy()), f32_bits(Y.cpu().numpy()))


def test_gemm_split_k_small_workspace_falls_back():
    M, N, K = 700, 3000, 4000
    note(f"gemm split-K short workspace M={M} N={N} K={K}")
    W = synth.gaussian((N, K), 9151, 0.02)
    X = synth.gaussian((M, K), 9651)
    pw, q = gpu_pack(W), gpu_quant(X)
    short = torch.zeros(bt.gemm_workspace_bytes(M, N, K) - 256, dtype=torch.uint8, device=DEV)
    short.fill_(0xFF)  # never read: too small for the split route
    Y1, a1 = bt.ternary_gemm(pw, q, want_acc=True)
    Y2, a2 = bt.ternary_gemm(pw, q, want_acc=True, workspace=short)
    np.testing.assert_array_equal(a1.cpu().numpy(), a2.cpu().numpy())
    np.testing.assert_array_equal(f32_bits(Y1.cpu().numpy()), f32_bits(Y2.cpu().numpy()))


@pytest.mark.parametrize("M,j,kernel", [(256, 0, "k_gemm_ks"), (256, 1, "k_gemm_ks"), (256, 3, "k_gemm_ks"),
                                        (2048, 3, "k_gemm<SPLITK=1")])
def test_2b_prefill_routed_shapes(M, j, kernel):
    """The 2B prefill shapes that take the small-M form (M=256: QKV, O, down) or split their
    last round (M=2048: down), in the launch configuration the benchmark times: sampled rows
    against the oracle, every output bit-identical to the call without a workspace."""
    name, N, K = synth.SHAPES_2B[j]
    note(f"2B prefill M={M} {name} ({kernel})")
    assert bt.kernel_plan(bt.CALL_GEMM_WS, M, N, K).startswith(kernel)
    W = synth.layer_weight(synth.CFG_2B_PREFILL, 0, j, N, K)
    X = synth.layer_activation(synth.CFG_2B_PREFILL, j, M, K)
    g = oracle.absmean(W)
    T = oracle.ternarize(W, g)
    Q, s, qs = oracle.quant_act(X)
    rows = np.concatenate([np.arange(0, M, 37), [M - 1]])
    acc_ref = oracle.ternary_matmul(T, Q[rows])
    pw, q = gpu_pack(W), gpu_quant(X)
    ws = bt.gemm_workspace(M, N, K, DEV)
    Y, acc = bt.ternary_gemm(pw, q, want_acc=True, workspace=ws)
    np.testing.assert_array_equal(acc.cpu().numpy()[rows], acc_ref)
    assert tol_ok(Y.cpu().numpy()[rows], oracle.scale_epilogue(acc_ref, g, s[rows]))
    Y1, a1 = bt.ternary_gemm(pw, q, want_acc=True)
    np.testing.assert_array_equal(a1.cpu().numpy(), acc.cpu().numpy())
    np.testing.assert_array_equal(f32_bits(Y1.cpu().numpy()), f32_bits(Y.cpu().numpy()))
    assert counters_zero(ws, M, N, K)


def test_2b_prefill_m2048_gate_up_sampled():
    note("2B prefill M=2048 gate_up")
    j = 2
    name, N, K = synth.SHAPES_2B[j]
    W = synth.layer_weight(synth.CFG_2B_PREFILL, 0, j, N, K)
    X = synth.layer_activation(synth.CFG_2B_PREFILL, j, 2048, K)
    g = oracle.absmean(W)
    T = oracle.ternarize(W, g)
    Q, s, qs = oracle.quant_act(X)
    rows = np.concatenate([np.arange(0, 2048, 61), [2047]])
    acc_ref = oracle.ternary_matmul(T, Q[rows])
    pw, q = gpu_pack(W), gpu_quant(X)
    Y, acc = bt.ternary_gemm(pw, q, want_acc=True)
    np.testing.assert_array_equal(acc.cpu().numpy()[rows], acc_ref)
    assert tol_ok(Y.cpu().numpy()[rows], oracle.scale_epilogue(acc_ref, g, s[rows]))


# ------------------------------------------------ invariants and edges
def test_negated_weights_negate_y_bitwise():
    note("negate W")
    W = synth.gaussian((300, 700), 9900, 0.02)
    X = synth.gaussian((4, 700), 9901)
    q = gpu_quant(X)
    Y1, a1 = bt.ternary_gemv(gpu_pack(W), q, want_acc=True)
    Y2, a2 = bt.ternary_gemv(gpu_pack(-W), q, want_acc=True)
    np.testing.assert_array_equal(a2.cpu().numpy(), -a1.cpu().numpy())
    np.testing.assert_array_equal(Y2.cpu().numpy(), -Y1.cpu().numpy())


def test_zero_weights_and_empty_k():
    note("zero W / K=0")
    X = synth.gaussian((3, 100), 9902)
    Y, acc = bt.ternary_gemv(gpu_pack(np.zeros((70, 100), np.float32)), gpu_quant(X), want_acc=True)
    assert not acc.cpu().numpy().any() and not Y.cpu().numpy().any()
    # K = 0: every accumulator is an empty sum
    W0 = torch.zeros((70, 0), dtype=torch.float32, device=DEV)
    pw0 = bt.pack_weights(W0)
    q0 = bt.quant_act(torch.zeros((3, 0), dtype=torch.float32, device=DEV))
    for fn in (bt.ternary_gemv, bt.ternary_gemm):
        Y, acc = fn(pw0, q0, want_acc=True)
        assert not acc.cpu().numpy().any() and not Y.cpu().numpy().any()


def test_outputs_optional():
    note("optional outputs")
    W = synth.gaussian((128, 256), 9903, 0.02)
    X = synth.gaussian((2, 256), 9904)
    ref = oracle_layer(W, X)
    pw, q = gpu_pack(W), gpu_quant(X)
    Y, acc = bt.ternary_gemv(pw, q, want_y=False, want_acc=True)
    assert Y is None
    np.testing.assert_array_equal(acc.cpu().numpy(), ref["acc"])
    Y, acc = bt.ternary_gemm(pw, q, want_y=True, want_acc=False)
    assert acc is None and tol_ok(Y.cpu().numpy(), ref["Y"])


def test_error_paths_raise():
    note("errors")
    W = synth.gaussian((64, 64), 9905, 0.02)
    X = synth.gaussian((17, 64), 9906)
    pw, q = gpu_pack(W), gpu_quant(X)
    with pytest.raises(bt.BTError) as e:
        bt.ternary_gemv(pw, q)
    assert e.value.name == "BT_ERR_UNSUPPORTED"


def test_side_stream_and_graph_replay():
    """Work enqueued on a non-default stream and captured in a HIP graph, replayed with new inputs."""
    note("stream + graph")
    N, K, M = 3840, 2560, 1
    W = synth.gaussian((N, K), 9907, 0.02)
    pw = gpu_pack(W)
    T = oracle.ternarize(W, oracle.absmean(W))
    xin = torch.zeros((M, K), dtype=torch.float32, device=DEV)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        q = bt.quant_act(xin)
        Y, acc = bt.ternary_gemv(pw, q, want_acc=True)
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        bt.quant_act(xin, out=q)
        bt.ternary_gemv(pw, q, out_y=Y, out_acc=acc)
    for rep in range(3):
        X = synth.gaussian((M, K), 9910 + rep)
        xin.copy_(to_dev(X))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        Q, sx, qs = oracle.quant_act(X)
        acc_ref = oracle.ternary_matmul(T, Q)
        np.testing.assert_array_equal(acc.cpu().numpy(), acc_ref)
        eager_Y, eager_acc = bt.ternary_gemv(pw, bt.quant_act(to_dev(X)), want_acc=True)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(Y.cpu().numpy(), eager_Y.cpu().numpy())


# ------------------------------------------------- fused linear entry point
# Shapes the fused kernel takes (M <= 4 and M * K <= 32768), token counts 1, 2 and 4
# (the kernel's three token capacities), ragged and aligned K.
LINEAR_CASES = [(1, 1, 1), (1, 100, 300), (2, 130, 129), (3, 65, 1000), (4, 200, 700), (4, 64, 64),
                (4, 300, 517), (4, 1000, 2560), (1, 2560, 6912), (1, 600, 28672), (4, 4096, 8192),
                # several tokens with fewer k-splits: S = 2 (four row blocks per workgroup),
                # S = 1 (eight), S = 4 (two)
                (4, 9000, 1000), (2, 20000, 520), (3, 8192, 1000)]


@pytest.mark.parametrize("M,N,K", LINEAR_CASES)
def test_linear_fused(M, N, K):
    """bt_ternary_linear (quantizer fused into the decode kernel) against the oracle, and bit-identical
    to the split route bt_quant_act + bt_ternary_gemv."""
    note(f"linear M={M} N={N} K={K}")
    assert bt.linear_workspace_bytes(M, N, K) == 0  # these shapes take the fused kernel
    W = synth.gaussian((N, K), 9200 + N + K, 0.02)
    X = synth.gaussian((M, K), 9700 + M + K)
    if M >= 3:
        X[1] = 0.0
    ref = oracle_layer(W, X)
    pw = gpu_pack(W)
    Y, acc = bt.linear(to_dev(X), pw, want_acc=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(acc.cpu().numpy(), ref["acc"])
    assert tol_ok(Y.cpu().numpy(), ref["Y"])
    Ys, _ = bt.ternary_gemv(pw, gpu_quant(X), algo=bt.GEMV_MFMA)
    np.testing.assert_array_equal(Y.cpu().numpy(), Ys.cpu().numpy())


@pytest.mark.parametrize("M,N,K", [(1, 3840, 2560), (4, 300, 1000), (8, 2560, 6912), (16, 1000, 2560)])
@pytest.mark.parametrize("shift_y,shift_acc", [(1, 0), (0, 3), (2, 2)])
def test_linear_outputs_not_16_byte_aligned(M, N, K, shift_y, shift_acc):
    """Caller outputs that start 4, 8 or 12 bytes past a 16-byte boundary (views into larger
    buffers) on the decode routes (fused at 1 and 4 tokens, quantizer + staged product at 8
    and 16): their four-output stores fall back to element stores; the results match the
    oracle and no element outside the views is written."""
    note(f"linear unaligned outputs M={M} N={N} K={K} shifts {shift_y} {shift_acc}")
    W = synth.gaussian((N, K), 9400 + N + K, 0.02)
    X = synth.gaussian((M, K), 9900 + M + K)
    ref = oracle_layer(W, X)
    ybuf = torch.full((M * N + 8,), 1234.5, dtype=torch.float32, device=DEV)
    abuf = torch.full((M * N + 8,), -7, dtype=torch.int32, device=DEV)
    Yv = ybuf[shift_y:shift_y + M * N].view(M, N)
    Av = abuf[shift_acc:shift_acc + M * N].view(M, N)
    bt.linear(to_dev(X), gpu_pack(W), out_y=Yv, out_acc=Av)
    torch.cuda.synchronize()
    bad = np.argwhere(Av.cpu().numpy() != ref["acc"])
    assert bad.size == 0, f"{len(bad)} acc mismatches, first at {bad[:5].tolist()}"
    assert tol_ok(Yv.cpu().numpy(), ref["Y"])
    yb, ab = ybuf.cpu().numpy(), abuf.cpu().numpy()
    assert (yb[:shift_y] == 1234.5).all() and (yb[shift_y + M * N:] == 1234.5).all()
    assert (ab[:shift_acc] == -7).all() and (ab[shift_acc + M * N:] == -7).all()


@pytest.mark.parametrize("M,N,K", [(1, 3840, 2560), (4, 300, 1000), (2, 600, 6912), (8, 500, 2560)])
def test_linear_misaligned_input(M, N, K):
    """Token rows at a 4-byte (not 16-byte) offset with K % 4 == 0: the fused kernel then reads
    them with scalar loads instead of its register path, the unfused route's quantizer likewise.
    Against the oracle, and bit-identical to the same call on an aligned copy (both entry points)."""
    note(f"linear misaligned input M={M} N={N} K={K}")
    W = synth.gaussian((N, K), 9400 + N + K, 0.02)
    X = synth.gaussian((M, K), 9900 + M + K)
    ref = oracle_layer(W, X)
    pw = gpu_pack(W)
    big = torch.zeros(X.size + 1, dtype=torch.float32, device=DEV)
    big[1:] = to_dev(X.ravel())
    Xd = big[1:].view(M, K)
    assert Xd.data_ptr() % 16 == 4
    Y, acc = bt.linear(Xd, pw, want_acc=True)
    Ys, accs = bt.linear_static(Xd, pw, want_acc=True)
    Ya, acca = bt.linear(to_dev(X), pw, want_acc=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(acc.cpu().numpy(), ref["acc"])
    assert tol_ok(Y.cpu().numpy(), ref["Y"])
    for y, a in ((Ys, accs), (Ya, acca)):
        np.testing.assert_array_equal(a.cpu().numpy(), ref["acc"])
        np.testing.assert_array_equal(f32_bits(y.cpu().numpy()), f32_bits(Y.cpu().numpy()))


@pytest.mark.parametrize("M,N,K", [(16, 512, 8192), (16, 600, 28672), (40, 300, 700), (300, 257, 1000),
                                   (5, 200, 700), (8, 64, 64), (16, 300, 517), (16, 1000, 2560),
                                   (8, 4096, 4096), (4, 300, 11008)])
def test_linear_workspace_routes(M, N, K):
    """Shapes outside the fused kernel's range (M > 4, M * K > 32768, M > 16) go through the
    workspace route: bt_quant_act, then bt_ternary_gemv or bt_ternary_gemm."""
    note(f"linear route M={M} N={N} K={K}")
    assert bt.linear_workspace_bytes(M, N, K) > 0
    W = synth.gaussian((N, K), 9300 + N, 0.02)
    X = synth.gaussian((M, K), 9800 + M)
    ref = oracle_layer(W, X)
    Y, acc = bt.linear(to_dev(X), gpu_pack(W), want_acc=True)
    np.testing.assert_array_equal(acc.cpu().numpy(), ref["acc"])
    assert tol_ok(Y.cpu().numpy(), ref["Y"])


def test_linear_tail_split_garbage_workspace():
    """bt_ternary_linear on a shape whose GEMM splits only its last tiles, with a workspace
    full of garbage: sampled rows against the oracle, all outputs bit-identical to the
    unsplit product."""
    M, N, K = 1100, 4096, 6200
    note(f"linear tail split garbage workspace M={M} N={N} K={K}")
    assert bt.gemm_split_plan(M, N, K) == (256, 4)
    W = synth.gaussian((N, K), 9153, 0.02)
    X = synth.gaussian((M, K), 9653)
    g = oracle.absmean(W)
    T = oracle.ternarize(W, g)
    Q, s, qs = oracle.quant_act(X)
    rows = np.concatenate([np.arange(7, M, 67), [M - 1]])
    acc_ref = oracle.ternary_matmul(T, Q[rows])
    pw = gpu_pack(W)
    ws = torch.full((bt.linear_workspace_bytes(M, N, K),), 0xFF, dtype=torch.uint8, device=DEV)
    for _ in range(2):
        Y, acc = bt.linear(to_dev(X), pw, want_acc=True, workspace=ws)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(acc.cpu().numpy()[rows], acc_ref)
        assert tol_ok(Y.cpu().numpy()[rows], oracle.scale_epilogue(acc_ref, g, s[rows]))
    Y1, a1 = bt.ternary_gemm(pw, gpu_quant(X), want_acc=True)
    np.testing.assert_array_equal(a1.cpu().numpy(), acc.cpu().numpy())
    np.testing.assert_array_equal(f32_bits(Y1.cpu().numpy()), f32_bits(Y.cpu().numpy()))


def test_linear_split_k_garbage_workspace():
    """bt_ternary_linear on a shape whose GEMM splits K, with a workspace full of garbage:
    the call initializes everything it reads (the quantizer zero-fills the counters)."""
    M, N, K = 650, 3300, 5500
    note(f"linear split-K garbage workspace M={M} N={N} K={K}")
    assert split_of(M, N, K) == 3
    W = synth.gaussian((N, K), 9152, 0.02)
    X = synth.gaussian((M, K), 9652)
    g = oracle.absmean(W)
    T = oracle.ternarize(W, g)
    Q, s, qs = oracle.quant_act(X)
    rows = sampled_rows(M)
    acc_ref = oracle.ternary_matmul(T, Q[rows])
    pw = gpu_pack(W)
    ws = torch.full((bt.linear_workspace_bytes(M, N, K),), 0xFF, dtype=torch.uint8, device=DEV)
    for _ in range(2):
        Y, acc = bt.linear(to_dev(X), pw, want_acc=True, workspace=ws)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(acc.cpu().numpy()[rows], acc_ref)
        assert tol_ok(Y.cpu().numpy()[rows], oracle.scale_epilogue(acc_ref, g, s[rows]))


@pytest.mark.parametrize("j,name,N,K", [(j, *s) for j, s in enumerate(synth.SHAPES_2B)])
def test_linear_2b_decode_full(j, name, N, K):
    """The benchmark's call: fused bt_ternary_linear at M=1 on the 2B decode shapes, every output."""
    note(f"linear 2B {name}")
    W = synth.layer_weight(synth.CFG_2B_DECODE, 1, j, N, K)
    X = synth.layer_activation(synth.CFG_2B_DECODE, j, 1, K)
    ref = oracle_layer(W, X)
    Y, acc = bt.linear(to_dev(X), gpu_pack(W), want_acc=True)
    np.testing.assert_array_equal(acc.cpu().numpy(), ref["acc"])
    assert tol_ok(Y.cpu().numpy(), ref["Y"])


def test_linear_100b_gate_up_m1_sampled():
    """Largest decode matrix (57344 x 8192, 117 MB packed) through the fused call, sampled rows."""
    note("linear 100B gate_up")
    j = 2
    name, N, K = synth.SHAPES_100B[j]
    W = synth.layer_weight(synth.CFG_100B_DECODE, 0, j, N, K)
    X = synth.layer_activation(synth.CFG_100B_DECODE, j, 1, K)
    g = oracle.absmean(W)
    rows = np.arange(0, N, 13)
    T = oracle.ternarize(W[rows], g)
    Q, s, qs = oracle.quant_act(X)
    acc_ref = oracle.ternary_matmul(T, Q)
    pw = gpu_pack(W)
    del W
    assert f32_bits(pw.scale.cpu().numpy()[0]) == f32_bits(g)
    Y, acc = bt.linear(to_dev(X), pw, want_acc=True)
    np.testing.assert_array_equal(acc.cpu().numpy()[:, rows], acc_ref)
    assert tol_ok(Y.cpu().numpy()[:, rows], oracle.scale_epilogue(acc_ref, g, s))


# ------------------------------------------------------- table-lookup GEMV (M = 1)
def _lut_fits(K):
    props = torch.cuda.get_device_properties(0)
    limit = getattr(props, "shared_memory_per_block", 65536)
    return ((K + 63) // 64) * 1024 + 1024 <= limit


@pytest.mark.parametrize("N,K", [(1, 1), (100, 300), (65, 129), (17, 64), (3840, 2560), (2560, 2560),
                                 (13824, 2560), (2560, 6912), (12288, 4096)])
def test_gemv_lut(N, K):
    """BT_GEMV_LUT (tables of code-pair sums in LDS) against the oracle and bit-identical to MFMA."""
    note(f"gemv lut N={N} K={K}")
    if not _lut_fits(K):
        pytest.skip(f"LUT tables for K = {K} exceed this device's per-workgroup LDS")
    W = synth.gaussian((N, K), 9900 + N + K, 0.02)
    X = synth.gaussian((1, K), 9950 + K)
    ref = oracle_layer(W, X)
    pw = gpu_pack(W)
    q = gpu_quant(X)
    check_product(pw, q, ref, 1, N, bt.ternary_gemv, algo=bt.GEMV_LUT)
    Y2, acc2 = bt.ternary_gemv(pw, q, want_acc=True, algo=bt.GEMV_MFMA)
    Y1, acc1 = bt.ternary_gemv(pw, q, want_acc=True, algo=bt.GEMV_LUT)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(acc1.cpu().numpy(), acc2.cpu().numpy())
    np.testing.assert_array_equal(Y1.cpu().numpy(), Y2.cpu().numpy())


def test_gemv_lut_row_scales_and_limits():
    note("gemv lut row scales / limits")
    N, K, groups = 768, 700, [640, 64, 64]
    W = synth.gaussian((N, K), 9960, 0.02)
    W[640:704] *= np.float32(9.0)
    X = synth.gaussian((1, K), 9961)
    ref = oracle.linear_rows(W, X, groups)
    pw = bt.pack_weights_rows(to_dev(W), groups)
    Y, acc = bt.ternary_gemv(pw, bt.quant_act(to_dev(X)), want_acc=True, algo=bt.GEMV_LUT)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(acc.cpu().numpy(), ref["acc"])
    assert tol_ok(Y.cpu().numpy(), ref["Y"])
    # two tokens: the LUT kernel takes one
    X2 = synth.gaussian((2, K), 9962)
    with pytest.raises(bt.BTError):
        bt.ternary_gemv(gpu_pack(W), gpu_quant(X2), algo=bt.GEMV_LUT)


# ------------------------------------------------- staged GEMV (5 <= M <= 16 tokens)
STAGED_CASES = [(5, 100, 300), (8, 130, 129), (8, 4096, 4096), (12, 600, 2560), (16, 2560, 1000),
                (16, 13824, 2560), (7, 20000, 520), (16, 65, 4096), (1, 3840, 2560), (4, 300, 517),
                # four chunks per thread: above 64 KB of staged rows, up to the 128 KB limit
                (16, 10240, 8192), (9, 300, 11008),
                # degenerate and maximum shapes: one column, one row, K = BT_MAX_K at one token,
                # and 128 KB of staged rows at two tokens
                (16, 70, 1), (16, 1, 300), (1, 70, 131072), (2, 33, 65536)]


@pytest.mark.parametrize("M,N,K", STAGED_CASES)
def test_gemv_staged(M, N, K):
    """BT_GEMV_STAGED (int8 rows staged in LDS) against the oracle and bit-identical to the direct MFMA kernel."""
    note(f"gemv staged M={M} N={N} K={K}")
    W = synth.gaussian((N, K), 9800 + N + K, 0.02)
    X = synth.gaussian((M, K), 9850 + M + K)
    if M >= 3:
        X[1] = 0.0
    ref = oracle_layer(W, X)
    pw = gpu_pack(W)
    q = gpu_quant(X)
    check_product(pw, q, ref, M, N, bt.ternary_gemv, algo=bt.GEMV_STAGED)
    Y1, acc1 = bt.ternary_gemv(pw, q, want_acc=True, algo=bt.GEMV_STAGED)
    Y2, acc2 = bt.ternary_gemv(pw, q, want_acc=True, algo=bt.GEMV_MFMA)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(acc1.cpu().numpy(), acc2.cpu().numpy())
    np.testing.assert_array_equal(Y1.cpu().numpy(), Y2.cpu().numpy())


# Rows too long to stage whole (M * K rounded up to 256 above 128 KB): the blocked form,
# which stages them in K-blocks of 2 S U steps. The k-splits S = 8, 4, 2, 1 (N) and token
# capacities 8 and 16 (M) cover every (S, U) pick; K ragged, K spanning a partial last block,
# and the 100B-class down shape at 5, 8 and 16 tokens.
BLOCKED_CASES = [(16, 64, 8448), (16, 2560, 28672), (5, 8192, 28672), (8, 8192, 28672), (16, 8192, 28672),
                 (9, 4096, 16000), (16, 20000, 8450), (12, 9000, 11008), (6, 4096, 22000), (16, 300, 131072)]


@pytest.mark.parametrize("M,N,K", BLOCKED_CASES)
def test_gemv_blocked(M, N, K):
    """BT_GEMV_STAGED (and BT_GEMV_AUTO) on rows staged in K-blocks, against the oracle (all rows up
    to 10000, else sampled) and bit-identical to the direct MFMA kernel."""
    plan = bt.kernel_plan(bt.CALL_GEMV, M, N, K, bt.GEMV_STAGED)
    note(f"gemv blocked M={M} N={N} K={K} plan={plan}")
    assert plan.startswith("k_gemv_blocked") and plan == bt.kernel_plan(bt.CALL_GEMV, M, N, K)
    W = synth.gaussian((N, K), 9880 + N + K, 0.02)
    X = synth.gaussian((M, K), 9890 + M + K)
    if M >= 3:
        X[1] = 0.0
    pw = gpu_pack(W)
    q = gpu_quant(X)
    Y1, acc1 = bt.ternary_gemv(pw, q, want_acc=True, algo=bt.GEMV_STAGED)
    Y2, acc2 = bt.ternary_gemv(pw, q, want_acc=True, algo=bt.GEMV_MFMA)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(acc1.cpu().numpy(), acc2.cpu().numpy())
    np.testing.assert_array_equal(Y1.cpu().numpy(), Y2.cpu().numpy())
    # gamma is the whole matrix's; the codes and products of the compared rows
    rows = np.arange(N) if N <= 10000 else np.unique(np.concatenate([np.arange(0, N, 97), [N - 1]]))
    g = oracle.absmean(W)
    Q, sx, _ = oracle.quant_act(X)
    acc_ref = oracle.ternary_matmul(oracle.ternarize(W[rows], g), Q)
    np.testing.assert_array_equal(acc1.cpu().numpy()[:, rows], acc_ref)
    assert tol_ok(Y1.cpu().numpy()[:, rows], oracle.scale_epilogue(acc_ref, g, sx))


def test_gemv_staged_limits_and_row_scales():
    note("gemv staged limits / row scales")
    # 16 tokens x 8448 columns of int8 would need 132 KB of LDS whole: the explicit staged
    # choice and BT_GEMV_AUTO both take the blocked form
    W = synth.gaussian((64, 8448), 9900, 0.02)
    X = synth.gaussian((16, 8448), 9901)
    pw, q = gpu_pack(W), gpu_quant(X)
    ref = oracle_layer(W, X)
    check_product(pw, q, ref, 16, 64, bt.ternary_gemv, algo=bt.GEMV_STAGED)
    check_product(pw, q, ref, 16, 64, bt.ternary_gemv, algo=bt.GEMV_AUTO)
    # the blocked form with row scales
    N, K, groups = 768, 9000, [640, 64, 64]
    W = synth.gaussian((N, K), 9904, 0.02)
    W[640:704] *= np.float32(5.0)
    X = synth.gaussian((16, K), 9905)
    ref = oracle.linear_rows(W, X, groups)
    pw = bt.pack_weights_rows(to_dev(W), groups)
    Y, acc = bt.ternary_gemv(pw, bt.quant_act(to_dev(X)), want_acc=True, algo=bt.GEMV_STAGED)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(acc.cpu().numpy(), ref["acc"])
    assert tol_ok(Y.cpu().numpy(), ref["Y"])
    # row scales
    N, K, groups = 768, 700, [640, 64, 64]
    W = synth.gaussian((N, K), 9902, 0.02)
    W[640:704] *= np.float32(5.0)
    X = synth.gaussian((9, K), 9903)
    ref = oracle.linear_rows(W, X, groups)
    pw = bt.pack_weights_rows(to_dev(W), groups)
    Y, acc = bt.ternary_gemv(pw, bt.quant_act(to_dev(X)), want_acc=True, algo=bt.GEMV_STAGED)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(acc.cpu().numpy(), ref["acc"])
    assert tol_ok(Y.cpu().numpy(), ref["Y"])
