"""Planted mistakes in a copy of the oracle's C source must fail the pins.

Each mutant is a text substitution in a temporary copy of moe_oracle.c, built
with gcc into a temporary directory; the committed oracle is never modified.
"""

import os
import subprocess

import pytest

import oracle
import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "moe_oracle.c")

MUTANTS = {
    "high_nibble_first": ("(4 * (c % 8))", "(4 * (7 - c % 8))"),
    "bias_dropped": ("* (double)q + bf16_to_double(m->B[g])", "* (double)q"),
    "scale_group_shifted": ("long g = row * (K / m->gs) + c / m->gs;",
                            "long g = row * (K / m->gs) + ((c / m->gs) + 1) % (K / m->gs);"),
    "gate_up_swapped": ("return silu(g) * u;", "return silu(u) * g;"),
    "router_weight_dropped": ("acc += (double)tw[t * k + j] * y[(t * k + j) * H + m];",
                              "acc += y[(t * k + j) * H + m];"),
    "token_index_wrong": ("pair_hidden_row(&bk, x + (p / k) * H, ids[p], H, I, n)",
                          "pair_hidden_row(&bk, x + (p % L) * H, ids[p], H, I, n)"),
    "down_uses_wrong_expert": ("y[pm] = pair_down_row(&bk, h + p * I, ids[p], H, I, m);",
                               "y[pm] = pair_down_row(&bk, h + p * I, ids[(p + 1) % P], H, I, m);"),
    "silu_wrong": ("return v / (1.0 + exp(-v));", "return v / (1.0 + exp(v));"),
}

PIN_TESTS = [
    pins.test_nibble_order_known_pattern,
    pins.test_scale_bias_roles_and_group_axis,
    pins.test_dense_swiglu_special_case_matches_library,
    lambda: pins.test_multi_expert_brute_force_matches_library(0),
    pins.test_closed_form_saturated_silu_integers,
    pins.test_gate_goes_through_silu_not_up,
]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, name
    mut = tmp_path / "mutant.c"
    mut.write_text(src.replace(old, new))
    so = str(tmp_path / "libmutant.so")
    subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-o", so, str(mut), "-lm"], check=True)
    prev = oracle.use_library(so)
    failed = []
    try:
        for t in PIN_TESTS:
            try:
                t()
            except AssertionError:
                failed.append(getattr(t, "__name__", "brute_force"))
    finally:
        oracle.restore_library(prev)
    assert failed, f"mutant {name} passed every pin"


# planted mistakes in the mxfp4 decode, against the mxfp4 pins
import test_oracle_mx_pins as mxpins  # noqa: E402

MX_MUTANTS = {
    "e2m1_exponent_bias_2": ("(int)expo - 1);", "(int)expo - 2);"),
    "e2m1_mantissa_quarter": ("ldexp(1.0 + 0.5 * (double)mant", "ldexp(1.0 + 0.25 * (double)mant"),
    "e2m1_sign_ignored": ("return sign ? -mag : mag;", "return mag;"),
    "e2m1_subnormal_step_1": ("expo == 0 ? 0.5 * (double)mant", "expo == 0 ? 1.0 * (double)mant"),
    "e8m0_bias_128": ("(int)e - 127);", "(int)e - 128);"),
    "mx_block_of_64": ("S[row * (K / 32) + c / 32]", "S[row * (K / 32) + c / 64]"),
}

MX_PIN_TESTS = [
    mxpins.test_code_table_closed_form_properties,
    mxpins.test_scale_byte_is_a_power_of_two_per_block,
    mxpins.test_grid_values_roundtrip_through_quantizer_and_decoder,
]


@pytest.mark.parametrize("name", sorted(MX_MUTANTS))
def test_mx_mutant_is_caught(name, tmp_path):
    old, new = MX_MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, name
    mut = tmp_path / "mutant.c"
    mut.write_text(src.replace(old, new))
    so = str(tmp_path / "libmutant.so")
    subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-o", so, str(mut), "-lm"], check=True)
    prev = oracle.use_library(so)
    failed = []
    try:
        for t in MX_PIN_TESTS:
            try:
                t()
            except AssertionError:
                failed.append(t.__name__)
    finally:
        oracle.restore_library(prev)
    assert failed, f"mutant {name} passed every mxfp4 pin"


# planted mistakes in the further codecs, against the codec pins
import test_oracle_codec_pins as cpins  # noqa: E402

CODEC_MUTANTS = {
    "e4m3_exponent_bias_8": ("(int)expo - 7);", "(int)expo - 8);"),
    "e4m3_subnormal_step": ("ldexp((double)mant / 8.0, -6)", "ldexp((double)mant / 8.0, -7)"),
    "e4m3_nan_lost": ("if (expo == 15u && mant == 7u) return NAN;", ""),
    "byte_order_reversed": ("(8 * (c % 4))", "(8 * (3 - c % 4))"),
    "nvfp4_block_of_32": ("S8[row * (K / 16) + c / 16]", "S8[row * (K / 16) + c / 32]"),
    "affine_group_fixed_64": ("long g = row * (K / m->gs) + c / m->gs;", "long g = row * (K / m->gs) + c / 64;"),
    "mxfp8_scale_bias_128": ("code8_at(m->W + row * (K / 4), c)), (int)e - 127);",
                             "code8_at(m->W + row * (K / 4), c)), (int)e - 128);"),
    "affine8_row_stride_of_4bit": ("m->W + row * (K * m->bits / 32)", "m->W + row * (K / 8)"),
}

CODEC_PIN_TESTS = [
    cpins.test_e4m3_decoder_matches_library_float8,
    cpins.test_known_code_patterns_decode_in_order,
    cpins.test_affine_group32_is_group64_with_repeated_scales,
    cpins.test_block_scales_act_on_their_own_block,
    cpins.test_grid_values_roundtrip_through_encoders_and_decoder,
]


@pytest.mark.parametrize("name", sorted(CODEC_MUTANTS))
def test_codec_mutant_is_caught(name, tmp_path):
    old, new = CODEC_MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, name
    mut = tmp_path / "mutant.c"
    mut.write_text(src.replace(old, new))
    so = str(tmp_path / "libmutant.so")
    subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-o", so, str(mut), "-lm"], check=True)
    prev = oracle.use_library(so)
    failed = []
    try:
        for t in CODEC_PIN_TESTS:
            try:
                t()
            except AssertionError:
                failed.append(t.__name__)
    finally:
        oracle.restore_library(prev)
    assert failed, f"mutant {name} passed every codec pin"
