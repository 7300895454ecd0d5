"""The CPU oracle built with AddressSanitizer and UndefinedBehaviorSanitizer.

tests/sanitize/oracle_driver.c runs the oracle's functions on cases read from a file, each
array in a heap block of exactly its documented size. Built with
-fsanitize=address,undefined (-fno-sanitize-recover), it runs a battery of the pins'
cases -- the hand-worked golden examples, the exhaustive ternary enumeration, the
reduction to an integer matmul, empty, single-element and ragged shapes, non-finite
inputs, row groups that do and do not cover the rows -- and must report nothing, return
the golden values, and agree bit for bit with the regular build of the oracle. CPU only.
"""
import json
import os
import shutil
import struct
import subprocess

import numpy as np
import pytest

import oracle
from bit_ternary_weight_absmean_amd import synth

HERE = os.path.dirname(os.path.abspath(__file__))
DRIVER = os.path.join(HERE, "sanitize", "oracle_driver.c")
GOLDEN = os.path.join(HERE, "golden", "hand_examples.json")
SAN_FLAGS = ["-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=all", "-fno-fast-math", "-ffp-contract=off"]
ENV = {"ASAN_OPTIONS": "detect_leaks=1:halt_on_error=1:abort_on_error=0",
       "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}

pytestmark = pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")


def _run_env():
    env = dict(os.environ)
    env.update(ENV)
    return env


@pytest.fixture(scope="module")
def san_driver(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("san") / "oracle_san")
    src = os.path.join(os.path.dirname(oracle.__file__), "bt_oracle.c")
    res = subprocess.run(["gcc", *SAN_FLAGS, DRIVER, src, "-lm", "-o", out], capture_output=True, text=True)
    if res.returncode != 0 and "fsanitize" in res.stderr:
        pytest.skip(f"the sanitizer runtimes are not available: {res.stderr[-300:]}")
    assert res.returncode == 0, res.stderr
    return out


def test_sanitizers_catch_a_planted_overflow(tmp_path):
    """The toolchain really reports: a one-past-the-end heap read built with the same flags."""
    src = tmp_path / "oob.c"
    src.write_text("#include <stdlib.h>\nint main(void){volatile int *p = malloc(4*sizeof(int));"
                   "int x = p[4]; free((void*)p); return x & 0;}\n")
    exe = str(tmp_path / "oob")
    res = subprocess.run(["gcc", *SAN_FLAGS, str(src), "-o", exe], capture_output=True, text=True)
    if res.returncode != 0 and "fsanitize" in res.stderr:
        pytest.skip("the sanitizer runtimes are not available")
    run = subprocess.run([exe], capture_output=True, text=True, env=_run_env())
    assert run.returncode != 0
    assert "heap-buffer-overflow" in run.stderr or "runtime error" in run.stderr, run.stderr[-500:]


class Cases:
    """Builds the case file and knows how to read each result back."""

    def __init__(self):
        self.buf = bytearray()
        self.expect = []  # (fn, dims, output spec, reference callable or value)

    def add(self, fn, dims, f, arrays, outs, ref):
        d = list(dims) + [0] * (3 - len(dims))
        self.buf += struct.pack("<iqqqf", fn, *d, float(f))
        for a in arrays:
            self.buf += np.ascontiguousarray(a).tobytes()
        self.expect.append((fn, outs, ref))

    def parse(self, raw):
        pos, got = 0, []
        for fn, outs, _ in self.expect:
            rc = struct.unpack_from("<i", raw, pos)[0]
            pos += 4
            vals = []
            for dtype, count in outs:
                n = np.dtype(dtype).itemsize * count
                vals.append(np.frombuffer(raw[pos:pos + n], dtype=dtype).copy())
                pos += n
            got.append((rc, vals))
        assert pos == len(raw), "results file longer than expected"
        return got


def _f32(a):
    return np.ascontiguousarray(a, np.float32)


def add_layer(cases, W, X):
    """absmean, ternarize, quant_act, matmul, epilogue on one (W, X), each checked against the
    regular oracle (and the golden values when given)."""
    W, X = _f32(W), _f32(X)
    N, K = W.shape
    M = X.shape[0]
    r = oracle.linear(W, X) if (N * K and M) else None
    g = oracle.absmean(W)
    cases.add(1, (N, K), 0, [W], [(np.float32, 1)], (0, [np.array([g], np.float32)]))
    T = oracle.ternarize(W, g)
    cases.add(2, (N, K), g, [W], [(np.int8, N * K)], (0, [T.ravel()]))
    Q, s, qs = oracle.quant_act(X)
    cases.add(3, (M, K), 0, [X], [(np.int8, M * K), (np.float32, M), (np.int32, M)],
              (0, [Q.ravel(), s, qs]))
    acc = oracle.ternary_matmul(T, Q)
    cases.add(4, (M, N, K), 0, [T, Q], [(np.int32, M * N)], (0, [acc.ravel()]))
    Y = oracle.scale_epilogue(acc, g, s)
    cases.add(5, (M, N), g, [acc, s], [(np.float32, M * N)], (0, [Y.ravel()]))
    return r


def build_cases():
    cases = Cases()
    golden = []
    # 1. the hand-worked golden examples
    with open(GOLDEN) as fh:
        for ex in json.load(fh)["examples"]:
            W = np.array(ex["W"], np.float32)
            X = np.array(ex["X"], np.float32)
            n0 = len(cases.expect)
            add_layer(cases, W, X)
            golden.append((n0, ex))
    # 2. random and degenerate shapes, ragged and aligned
    for i, (M, N, K) in enumerate([(1, 1, 1), (2, 3, 7), (4, 64, 64), (3, 100, 300), (5, 65, 129), (16, 37, 517),
                                   (1, 5, 0), (1, 0, 5), (0, 5, 5)]):
        W = synth.gaussian((N, K), 400 + i, 0.02)
        X = synth.gaussian((M, K), 500 + i)
        if M >= 3:
            X[1] = 0.0
        add_layer(cases, W, X)
    # 3. exhaustive: all 3^6 ternary 2 x 3 matrices stacked, against random integer tokens
    grid = np.array(np.meshgrid(*[[-1, 0, 1]] * 6, indexing="ij")).reshape(6, -1).T.astype(np.int8)
    T = np.ascontiguousarray(grid.reshape(-1, 3))  # 1458 rows of 3
    rng = np.random.default_rng(7)
    Q = rng.integers(-127, 128, size=(4, 3)).astype(np.int8)
    cases.add(4, (4, T.shape[0], 3), 0, [T, Q], [(np.int32, 4 * T.shape[0])],
              (0, [(Q.astype(np.int64) @ T.astype(np.int64).T).astype(np.int32).ravel()]))
    # 4. the integer special case: W = c T, integer tokens of absmax 127 -> a library matmul
    T2 = rng.integers(-1, 2, size=(40, 90)).astype(np.int8)
    X2 = rng.integers(-127, 128, size=(6, 90)).astype(np.float32)
    X2[:, 0] = 127.0
    r = add_layer(cases, np.float32(0.37) * T2.astype(np.float32), X2)
    assert np.array_equal(r["acc"], (X2.astype(np.int64) @ T2.astype(np.int64).T).astype(np.int32))
    # 5. non-finite inputs are rejected (return code 1) without touching memory out of bounds
    Wn = synth.gaussian((4, 9), 600, 0.02)
    Wn[2, 5] = np.nan
    cases.add(1, (4, 9), 0, [Wn], [(np.float32, 1)], (1, None))
    cases.add(2, (4, 9), 0.01, [Wn], [(np.int8, 36)], (1, None))
    Xn = synth.gaussian((3, 11), 601)
    Xn[1, 10] = np.inf
    cases.add(3, (3, 11), 0, [Xn], [(np.int8, 33), (np.float32, 3), (np.int32, 3)], (1, None))
    cases.add(9, (3, 11), 0, [Xn], [(np.float32, 3)], (1, None))
    cases.add(10, (3, 11), 0, [Xn], [(np.int8, 33)], (1, None))
    # 6. row groups: explicit groups, one group per row, groups that do not cover the rows
    Wr = synth.gaussian((10, 13), 602, 0.02)
    Wr[4:7] *= np.float32(8.0)
    for seg in ([4, 3, 3], [10], None):
        rs = oracle.absmean_rows(Wr, seg)
        segarr = np.array(seg or [], np.int64)
        cases.add(6, (10, 13, len(segarr)), 0, [Wr] + ([segarr] if len(segarr) else []), [(np.float32, 10)],
                  (0, [rs]))
        Tr = oracle.ternarize_rows(Wr, rs)
        cases.add(7, (10, 13), 0, [Wr, rs], [(np.int8, 130)], (0, [Tr.ravel()]))
        Xr = synth.gaussian((3, 13), 603)
        Qr, sr, _ = oracle.quant_act(Xr)
        accr = oracle.ternary_matmul(Tr, Qr)
        cases.add(8, (3, 10), 0, [accr, rs, sr], [(np.float32, 30)],
                  (0, [oracle.scale_epilogue_rows(accr, rs, sr).ravel()]))
    for bad in ([4, 7], [4, 5], [0, 10]):
        cases.add(6, (10, 13, len(bad)), 0, [Wr, np.array(bad, np.int64)], [(np.float32, 10)], (2, None))
    # 7. 1-bit operands: absmax per row and binarization (+0, -0, subnormals)
    V = synth.gaussian((5, 33), 604)
    V[0, :4] = [0.0, -0.0, 1e-45, -1e-45]
    cases.add(9, (5, 33), 0, [V], [(np.float32, 5)], (0, [oracle.absmax_rows(V)]))
    cases.add(10, (5, 33), 0, [V], [(np.int8, 165)], (0, [oracle.binarize(V).ravel()]))
    return cases, golden


def test_sanitized_oracle_battery(san_driver, tmp_path):
    cases, golden = build_cases()
    cin, cout = tmp_path / "cases.bin", tmp_path / "results.bin"
    cin.write_bytes(bytes(cases.buf))
    run = subprocess.run([san_driver, str(cin), str(cout)], capture_output=True, text=True, env=_run_env(),
                         timeout=600)
    assert run.returncode == 0, f"sanitized oracle failed ({run.returncode}):\n{run.stderr[-3000:]}"
    assert "runtime error" not in run.stderr and "AddressSanitizer" not in run.stderr, run.stderr[-3000:]
    got = cases.parse(cout.read_bytes())
    for i, ((rc, vals), (fn, _, (rc_ref, ref))) in enumerate(zip(got, cases.expect)):
        assert rc == rc_ref, f"case {i} (fn {fn}): return code {rc}, expected {rc_ref}"
        if ref is not None:
            for v, e in zip(vals, ref):
                e = np.asarray(e).ravel()
                assert np.array_equal(v.view(np.uint8), e.astype(v.dtype).view(np.uint8)), f"case {i} (fn {fn})"
    # the golden examples' values, read back from the sanitized build
    for n0, ex in golden:
        g = got[n0][1][0][0]
        assert g == np.float32(float.fromhex(ex["gamma"])), ex["name"]
        np.testing.assert_array_equal(got[n0 + 1][1][0], np.array(ex["T"], np.int8).ravel())
        np.testing.assert_array_equal(got[n0 + 2][1][0], np.array(ex["Q"], np.int8).ravel())
        np.testing.assert_array_equal(got[n0 + 3][1][0], np.array(ex["acc"], np.int32).ravel())


def test_sanitized_battery_catches_a_planted_oracle_overrun(tmp_path):
    """A copy of the oracle whose integer loop reads one k past the row (k <= K) must be
    reported by the sanitized battery: the battery exercises the oracle's memory bounds."""
    src = os.path.join(os.path.dirname(oracle.__file__), "bt_oracle.c")
    text = open(src).read()
    old = "for (int64_t k = 0; k < K; ++k)\n                s += (int32_t)T[n * K + k] * (int32_t)Q[m * K + k];"
    assert old in text
    bad = tmp_path / "bt_oracle_overrun.c"
    bad.write_text(text.replace(old, old.replace("k < K", "k <= K")))
    exe = str(tmp_path / "oracle_overrun")
    res = subprocess.run(["gcc", *SAN_FLAGS, DRIVER, str(bad), "-lm", "-o", exe], capture_output=True, text=True)
    if res.returncode != 0 and "fsanitize" in res.stderr:
        pytest.skip("the sanitizer runtimes are not available")
    assert res.returncode == 0, res.stderr
    cases, _ = build_cases()
    cin, cout = tmp_path / "cases.bin", tmp_path / "results.bin"
    cin.write_bytes(bytes(cases.buf))
    run = subprocess.run([exe, str(cin), str(cout)], capture_output=True, text=True, env=_run_env(), timeout=600)
    assert run.returncode != 0
    assert "heap-buffer-overflow" in run.stderr or "runtime error" in run.stderr, run.stderr[-500:]
