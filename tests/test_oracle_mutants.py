"""The oracle's pins must catch plausible mistakes.

Each mutant is a one-line edit of a temporary copy of the oracle's C source (the
committed oracle is untouched), compiled with the same gcc flags; the battery of pins
from test_oracle_pins must fail on every mutant. CPU only.
"""
import os
import subprocess

import numpy as np
import pytest

import oracle
import tests.test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "bt_oracle.c")

MUTANTS = {
    "threshold_gamma": ("const float half = gamma * 0.5f;", "const float half = gamma;"),
    "ties_to_nonzero": ("if (w > half)", "if (w >= half)"),
    "round_half_away": ("rintf(x[k] * inv)", "roundf(x[k] * inv)"),
    "round_truncate": ("rintf(x[k] * inv)", "truncf(x[k] * inv)"),
    "absmean_drops_last_k": ("for (int64_t k = 0; k < K; ++k) {\n            float w = W[n * K + k];",
                             "for (int64_t k = 0; k < K - 1; ++k) {\n            float w = W[n * K + k];"),
    "mean_without_abs": ("row += fabs((double)w);", "row += (double)w;"),
    "transposed_weight_index": ("(int32_t)T[n * K + k]", "(int32_t)T[k * N + n]"),
    "epilogue_drops_sx": ("(double)gamma * (double)s_x[m]);", "(double)gamma);"),
    "epilogue_drops_gamma": ("(double)acc[m * N + n] * (double)gamma", "(double)acc[m * N + n]"),
    "negative_code_sign": ("T[i] = -1;", "T[i] = 1;"),
    "int8_scale_128": ("const float inv = 127.0f / a;", "const float inv = 128.0f / a;"),
    "sx_inverted": ("s_x[m] = a / 127.0f;", "s_x[m] = 127.0f / a;"),
    "qsum_dropped": ("sum += (int32_t)r;", "(void)r;"),
    "rows_epilogue_token_index": ("(double)row_scale[n] * (double)s_x[m]", "(double)row_scale[m] * (double)s_x[m]"),
    "rows_group_from_first_row": ("if (oracle_absmean(W + n0 * K, rows, K, &g))",
                                  "if (oracle_absmean(W + n0 * K, 1, K, &g))"),
    "rows_codes_first_scale": ("row_scale[n], T + n * K", "row_scale[0], T + n * K"),
    "rows_group_start_stuck": ("        n0 += rows;\n    }\n    return n0 == N", "        n0 += 0;\n    }\n    return n0 == N"),
    "rows_epilogue_drops_scale": ("(double)acc[m * N + n] * (double)row_scale[n]", "(double)acc[m * N + n]"),
    "binarize_zero_negative": ("B[i] = V[i] >= 0.0f ? 1 : -1;", "B[i] = V[i] > 0.0f ? 1 : -1;"),
    "binarize_flipped": ("B[i] = V[i] >= 0.0f ? 1 : -1;", "B[i] = V[i] >= 0.0f ? -1 : 1;"),
    "absmax_keeps_min": ("if (fabsf(v) > a)", "if (fabsf(v) < a)"),
    "absmax_without_abs": ("if (fabsf(v) > a)\n                a = fabsf(v);", "if (v > a)\n                a = v;"),
}


def _battery(lib):
    """Run the pins against ``lib``; return the names of the pins that fail."""
    failed = []

    def run(name, fn, *args):
        try:
            fn(lib, *args)
        except (AssertionError, oracle.OracleInputError):
            failed.append(name)

    for ex in pins._EXAMPLES:
        run(ex["name"], pins.test_hand_examples, ex)
    for name in ("test_ternary_times_integer_is_library_matmul", "test_brute_force_1x4_rows_against_pm127_grid",
                 "test_add_subtract_skip_form", "test_gamma_is_exact_mean_rounded", "test_zero_fraction_gaussian",
                 "test_quant_rounding_bound_and_range", "test_quant_odd_and_scale_invariant",
                 "test_negating_w_negates_y", "test_y_equals_matmul_of_dequantized_operands",
                 "test_bitplane_popcount_form", "test_row_group_scales_are_exact_group_means",
                 "test_row_group_codes_gaussian_zero_fraction", "test_row_scales_power_of_two_rows",
                 "test_one_group_is_the_per_matrix_layer", "test_row_groups_equal_separate_matrices",
                 "test_binary_acc_is_the_pages_xnor_popcount", "test_ternary_a1_acc_is_the_pages_bitplane_form",
                 "test_binarize_signs_and_zero", "test_absmax_rows_is_numpy_max_abs",
                 "test_binary_layer_exact_when_magnitudes_are_constant"):
        run(name, getattr(pins, name))
    return failed


def test_unmutated_oracle_passes_battery(orc):
    assert _battery(orc) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    find, repl = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(find) == 1, f"mutation anchor for {name} not unique in the oracle source"
    mutated = tmp_path / "bt_oracle_mut.c"
    mutated.write_text(src.replace(find, repl))
    so = tmp_path / "liboracle_mut.so"
    subprocess.run(["gcc", *oracle.CFLAGS, "-o", str(so), str(mutated), "-lm"], check=True)
    lib = oracle.load(str(so))
    failed = _battery(lib)
    assert failed, f"mutant {name} survived every pin"
