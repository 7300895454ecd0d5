"""Every kernel instance the benchmark launches is also run by a GPU parity test.

bt_kernel_plan names the kernel instances (with their template arguments) that a call
launches. This test lists them for every step bench.py can time -- each workload at each
token count of bench.WORKLOAD_M, on the default route, ``--split`` and ``--row-scales`` --
and for the cases of the GPU parity modules, and checks that the first set lies inside the
second. It runs on the CPU: the query makes no device call.
"""
import re

import pytest

import bench
import bit_ternary_weight_absmean_amd as bt
from tests import test_parity_gpu as par
from tests import test_parity_routes_gpu as routes


def kernels(plan: str):
    """The kernel instances of a plan text. The GEMM's tile counts are reduced to the form of
    its work split (whole tiles, every tile split in S, or the last round split in S): the
    instance is the same kernel whatever the tile count."""
    out = []
    for k in plan.split(" + "):
        m = re.match(r"(k_gemm<[^>]*>)\[tiles=\d+(?:,full=(\d+),splits=(\d+))?\]", k)
        if m:
            if m.group(2) is None:
                k = m.group(1) + "[whole tiles]"
            elif m.group(2) == "0":
                k = m.group(1) + f"[every tile in {m.group(3)}]"
            else:
                k = m.group(1) + f"[last round in {m.group(3)}]"
        out.append(k)
    return out


def bench_instances():
    """{kernel instance: [where the benchmark launches it]}."""
    found = {}
    for workload, ms in bench.WORKLOAD_M.items():
        for m in ms:
            spec = bench.workload_spec(workload, m)
            for split in (False, True):
                for rows in (False, True):
                    for (name, N, K), plan in zip(spec["shapes"], bench.step_plans(spec, split, rows)):
                        flags = ("--split " if split else "") + ("--row-scales " if rows else "")
                        for k in kernels(plan):
                            found.setdefault(k, []).append(f"{workload} M={m} {name} {flags}".strip())
    return found


def parity_instances():
    """{kernel instance: [parity case that runs it]}."""
    found = {}

    def add(plan, case):
        for k in kernels(plan):
            found.setdefault(k, []).append(case)

    for workload, j, route in routes.route_cases():
        _, shapes, ms = routes.ROUTE_WORKLOADS[workload]
        name, N, K = shapes[j]
        for m in ms:
            add(routes.bench_plan(route, m, N, K, workload.endswith("prefill")),
                f"test_bench_route[{workload}-{j}-{route}] M={m}")
    for M, N, K in par.LINEAR_CASES:
        add(bt.kernel_plan(bt.CALL_LINEAR, M, N, K), f"test_linear_fused[{M}-{N}-{K}]")
    for M, N, K in par.STAGED_CASES:
        add(bt.kernel_plan(bt.CALL_GEMV, M, N, K, bt.GEMV_STAGED), f"test_gemv_staged[{M}-{N}-{K}]")
        add(bt.kernel_plan(bt.CALL_GEMV, M, N, K, bt.GEMV_MFMA), f"test_gemv_staged[{M}-{N}-{K}] (direct)")
    for M, N, K in par.GEMM_SMALL:
        add(bt.kernel_plan(bt.CALL_GEMM, M, N, K), f"test_gemm_small[{M}-{N}-{K}]")
    for M, N, K, _ in par.SPLIT_SHAPES:
        add(bt.kernel_plan(bt.CALL_GEMM_WS, M, N, K), f"test_gemm_split_k[{M}-{N}-{K}]")
    for M, N, K, _, _ in par.TAIL_SHAPES:
        add(bt.kernel_plan(bt.CALL_GEMM_WS, M, N, K), f"test_gemm_tail_split[{M}-{N}-{K}]")
    for M, K in par.QUANT_SHAPES:
        add(bt.kernel_plan(bt.CALL_QUANT, M, 1, K), f"test_quant_act[{M}-{K}]")
    return found


def test_routes_cover_the_bench_token_counts():
    """The route parity module runs each workload at the token counts bench.py is run at."""
    assert set(routes.ROUTE_WORKLOADS) == set(bench.WORKLOAD_M)
    for w, ms in bench.WORKLOAD_M.items():
        assert tuple(routes.ROUTE_WORKLOADS[w][2]) == tuple(ms), w


def test_every_bench_instance_has_a_parity_case():
    bench_k = bench_instances()
    par_k = parity_instances()
    missing = {k: v[:3] for k, v in bench_k.items() if k not in par_k}
    assert not missing, f"kernel instances the benchmark launches without a parity case: {missing}"


@pytest.mark.parametrize("plan,expect", [
    ("k_quant_act_reg<C=8> + k_gemm<SPLITK=1,ROWS=0>[tiles=320,full=256,splits=4]",
     ["k_quant_act_reg<C=8>", "k_gemm<SPLITK=1,ROWS=0>[last round in 4]"]),
    ("k_gemm<SPLITK=1,ROWS=1>[tiles=40,full=0,splits=3]", ["k_gemm<SPLITK=1,ROWS=1>[every tile in 3]"]),
    ("k_gemm<SPLITK=0,ROWS=0>[tiles=1728]", ["k_gemm<SPLITK=0,ROWS=0>[whole tiles]"]),
])
def test_plan_text_parsing(plan, expect):
    assert kernels(plan) == expect


def test_plan_query_errors():
    with pytest.raises(bt.BTError):
        bt.kernel_plan(bt.CALL_GEMV, 17, 64, 64)  # above the GEMV's token limit
    with pytest.raises(bt.BTError):
        bt.kernel_plan(bt.CALL_GEMV, 5, 64, 64, bt.GEMV_DOT4)
    with pytest.raises(bt.BTError):
        bt.kernel_plan(9, 1, 64, 64)
    assert bt.kernel_plan(bt.CALL_LINEAR, 0, 64, 64) == ""
    assert bt.kernel_plan(bt.CALL_LINEAR, 1, 3840, 2560).startswith("k_linear_decode<MT=1,")
