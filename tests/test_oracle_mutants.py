"""Planted mistakes in the oracle must be caught by its pins.

Each mutant is a copy of oracle/vq_oracle.c with one plausible slip (a sign,
a dropped term, a wrong index or stride, the wrong tie rule, a wrong group
mapping, a broken fp16 decode).  It is compiled on the CPU into a temporary
library, swapped in for the real one, and the pin tests are run against it:
at least one pin must fail for every mutant.
"""
import ctypes
import os
import subprocess
import tempfile

import pytest

import oracle
from tests import test_oracle_pins as pins
from tests import test_oracle_smooth_pack as sp

SRC = os.path.join(os.path.dirname(oracle.__file__), "vq_oracle.c")

MUTANTS = {
    "tie_keeps_last": ("if (dist < best) {\n                best = dist;\n                best_idx",
                       "if (dist <= best) {\n                best = dist;\n                best_idx"),
    "plus_instead_of_minus": ("widen(xrow[i], dtype) - widen(crow[i], dtype)",
                              "widen(xrow[i], dtype) + widen(crow[i], dtype)"),
    "dropped_last_term": ("for (int i = 0; i < sub_dim; ++i) {\n        float d",
                          "for (int i = 0; i + 1 < sub_dim; ++i) {\n        float d"),
    "abs_not_square": ("dist = fmaf(d, d, dist);", "dist = dist + fabsf(d);"),
    "row_stride_wrong": ("float dist = vqo_sqdist(xr, cb + (int64_t)c * sub_dim, sub_dim, dtype);\n            if (dist < best) {\n                best = dist;\n                best_idx = (uint32_t)c;\n            }\n        }\n        out[r] = best_idx;",
                         "float dist = vqo_sqdist(xr, cb + (int64_t)c, sub_dim, dtype);\n            if (dist < best) {\n                best = dist;\n                best_idx = (uint32_t)c;\n            }\n        }\n        out[r] = best_idx;"),
    "group_modulo": ("int64_t g = n / group_len;", "int64_t g = n % group_len;"),
    "slot_ignores_stride": ("const uint16_t *cb = codebook + slot * codebook_stride;\n        const uint16_t *xr = x + r * sub_dim;\n        float best = INFINITY;\n        uint32_t best_idx = 0;\n        for (int c = 0; c < n_centroids; ++c) {\n            float dist = vqo_sqdist(xr, cb + (int64_t)c * sub_dim, sub_dim, dtype);\n            if (dist < best) {\n                best = dist;\n                best_idx = (uint32_t)c;\n            }\n        }\n        out[r] = best_idx;",
                            "const uint16_t *cb = codebook + slot * (int64_t)n_centroids * sub_dim;\n        const uint16_t *xr = x + r * sub_dim;\n        float best = INFINITY;\n        uint32_t best_idx = 0;\n        for (int c = 0; c < n_centroids; ++c) {\n            float dist = vqo_sqdist(xr, cb + (int64_t)c * sub_dim, sub_dim, dtype);\n            if (dist < best) {\n                best = dist;\n                best_idx = (uint32_t)c;\n            }\n        }\n        out[r] = best_idx;"),
    "f16_bias_off_by_one": ("expo - 25);", "expo - 24);"),
    "f16_subnormal_scale": ("ldexpf((float)frac, -24)", "ldexpf((float)frac, -25)"),
    "start_index_last": ("float best = INFINITY;\n        uint32_t best_idx = 0;\n        for (int c = 0; c < n_centroids; ++c) {\n            float dist = vqo_sqdist(xr, cb + (int64_t)c * sub_dim, sub_dim, dtype);\n            if (dist < best) {\n                best = dist;\n                best_idx = (uint32_t)c;\n            }\n        }\n        out[r] = best_idx;",
                         "float best = INFINITY;\n        uint32_t best_idx = (uint32_t)(n_centroids - 1);\n        for (int c = 0; c < n_centroids; ++c) {\n            float dist = vqo_sqdist(xr, cb + (int64_t)c * sub_dim, sub_dim, dtype);\n            if (dist < best) {\n                best = dist;\n                best_idx = (uint32_t)c;\n            }\n        }\n        out[r] = best_idx;"),
    "decode_accepts_n_centroids": ("idx[r] >= (uint32_t)n_centroids", "idx[r] > (uint32_t)n_centroids"),
    "bf16_wrong_half": ("uint32_t u = (uint32_t)b << 16;", "uint32_t u = (uint32_t)b << 15;"),
    # smoothing, the fp32 search and the packed stream
    "pack_msb_first": ("out[bit / 8] |= (uint8_t)(b << (bit % 8));",
                       "out[bit / 8] |= (uint8_t)(b << (7 - bit % 8));"),
    "pack_drops_top_bit": ("for (int k = 0; k < code_bits; ++k) {\n            int64_t bit = r * code_bits + k;\n            uint32_t b",
                           "for (int k = 0; k + 1 < code_bits; ++k) {\n            int64_t bit = r * code_bits + k;\n            uint32_t b"),
    "smooth_channel_unscaled": ("const int64_t ch0 = (r % n_sub) * sub_dim;",
                                "const int64_t ch0 = (r % n_sub);"),
    "smooth_ignores_slot": ("channel_scale[slot * scale_stride + ch0 + i]", "channel_scale[ch0 + i]"),
    "smooth_adds": ("v = v * channel_scale[", "v = v + channel_scale["),
    "f32_search_plus": ("float d = xs[i] - widen(crow[i], dtype);",
                        "float d = xs[i] + widen(crow[i], dtype);"),
    "f32_bad_slot_zero": ("out[r] = VQO_BAD_SLOT;\n            if (best_out)",
                          "out[r] = 0;\n            if (best_out)"),
    "top2_second_counts_winner": ("if ((uint32_t)c == best_idx) continue;\n                float dist = sqdist_f32",
                                  "float dist = sqdist_f32"),
}

PIN_TESTS = [
    lambda: pins.test_f16_widening_matches_numpy_every_pattern(),
    lambda: pins.test_exact_grid_no_exemptions(oracle.F16),
    lambda: pins.test_exact_fp16_full_range(),
    lambda: pins.test_exact_bf16_range(),
    lambda: pins.test_x_equal_to_a_duplicated_centroid_gives_the_first_copy(),
    lambda: pins.test_equidistant_axis_rows_resolve_to_lowest_index(),
    lambda: pins.test_non_finite_inputs(),
    lambda: pins.test_sub_dim_one_equals_boundary_sum(),
    lambda: pins.test_group_slots_select_the_right_codebook(),
    lambda: pins.test_decode_gathers_rows_and_zeroes_bad_indices(),
    lambda: pins.test_bf16_widening_matches_torch_every_pattern(),
    lambda: sp.test_pack_golden_examples_from_the_pages(),
    lambda: [sp.test_pack_matches_numpy_little_endian_bits(b) for b in (1, 3, 8, 13, 32)],
    lambda: sp.test_smooth_matches_numpy_float32_multiply_in_cache_layout(),
    lambda: sp.test_power_of_two_factors_equal_encode_of_prescaled_keys(),
    lambda: sp.test_smoothed_search_against_exact_rational_brute_force(oracle.F16),
    lambda: sp.test_factor_vector_follows_the_codebook_slot(),
    lambda: sp.test_bad_slot_gets_all_ones_code_and_threads_agree(),
    lambda: sp.test_encode_f32_top2_second_is_the_runner_up(),
]


def _compile(src_text, tmp):
    c = os.path.join(tmp, "m.c")
    so = os.path.join(tmp, "m.so")
    with open(c, "w") as f:
        f.write(src_text)
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-shared", "-fPIC", c, "-o", so, "-lm"],
                   check=True, capture_output=True)
    return so


def _bind(so):
    saved = oracle._lib
    oracle._lib = None
    real = oracle._LIB_PATH
    oracle._LIB_PATH = so
    try:
        lib = oracle._load()
    finally:
        oracle._LIB_PATH = real
    return saved, lib


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name):
    src = open(SRC).read()
    old, new = MUTANTS[name]
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    mutated = src.replace(old, new, 1)
    with tempfile.TemporaryDirectory() as tmp:
        so = _compile(mutated, tmp)
        saved, _ = _bind(so)
        caught = False
        try:
            for pin in PIN_TESTS:
                try:
                    pin()
                except (AssertionError, ValueError):
                    caught = True
                    break
        finally:
            oracle._lib = saved
    assert caught, f"no pin caught the planted mistake {name!r}"


def test_unmutated_oracle_passes_the_same_pins():
    for pin in PIN_TESTS:
        pin()
