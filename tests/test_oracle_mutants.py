"""Planted mistakes in the oracle must fail at least one pin (no GPU).

Each mutant is a copy of ``oracle/q8_oracle.c`` with one plausible mistake
(a wrong constant, a dropped term, a wrong index or sign, a different
rounding reading), compiled with the oracle's own flags into a temporary
library.  The pins in ``pins.py`` are run against it; a mutant that passes
every pin would mean the pins cannot tell that mistake from the definition.
"""

import os

import pytest

import oracle
import pins

MUTANTS = {
    # quantisation
    "divisor_128": ("const float d = a / 127.0f;", "const float d = a / 128.0f;"),
    "round_half_even": ("float r = roundf(x[i] / d);", "float r = rintf(x[i] / d);"),
    "reciprocal_multiply": ("float r = roundf(x[i] / d);",
                            "float r = roundf(x[i] * (1.0f / d));"),
    "quantise_with_f16_scale": (
        "float r = roundf(x[i] / d);",
        "float r = roundf(x[i] / q8o_f16_to_f32(q8o_f32_to_f16(d)));"),
    "absmax_without_abs": ("const float v = fabsf(x[i]);", "const float v = x[i];"),
    "drop_sign": ("q[i] = (int8_t)r;", "q[i] = (int8_t)fabsf(r);"),
    "truncate": ("float r = roundf(x[i] / d);", "float r = truncf(x[i] / d);"),
    "nonfinite_quantised": ("        if (!(v <= FLT_MAX)) finite = 0; /* NaN or infinity */\n        else if",
                            "        if (0) finite = 0;\n        else if"),
    "nonfinite_inf_scale": ("        *d16 = 0x7e00u;", "        *d16 = 0x7c00u;"),
    "underflow_divides": ("    if (d == 0.0f) {", "    if (a == 0.0f) {"),
    # binary16 conversion
    "f16_ties_away": ("if (rem > half || (rem == half && (r & 1u))) r += 1u;",
                      "if (rem >= half) r += 1u;"),
    "f16_truncate": ("if (rem > half || (rem == half && (r & 1u))) r += 1u;",
                     "(void)half;"),
    "f16_subnormal_shift": ("const int s = -(E + 1);", "const int s = -(E + 2);"),
    "f16_bias": ("int E16 = E + 15;", "int E16 = E + 16;"),
    "f16_to_f32_subnormal": ("const float v = (float)m * 0x1p-24f;",
                             "const float v = (float)m * 0x1p-25f;"),
    # the matmul
    "dot_drops_last": ("for (int i = 0; i < Q8O_BLOCK; ++i) s += (int32_t)w[i] * (int32_t)x[i];",
                       "for (int i = 0; i < Q8O_BLOCK - 1; ++i) s += (int32_t)w[i] * (int32_t)x[i];"),
    "token_not_slot_q": ("qx + (int64_t)s * K + b * Q8O_BLOCK);\n                const double",
                         "qx + (int64_t)t * K + b * Q8O_BLOCK);\n                const double"),
    "token_not_slot_scale": ("dx[(int64_t)s * KB + b]", "dx[(int64_t)t * KB + b]"),
    "weight_scale_transposed": ("dw[n * KB + b]", "dw[b * N + n]"),
    "act_scale_dropped": ("(double)q8o_f16_to_f32(dx[(int64_t)s * KB + b]);",
                          "1.0;"),
    "float_accumulator": ("double y = 0.0, a = 0.0;", "float y = 0.0f; double a = 0.0;"),
    "abs_sum_signed": ("a += fabs(term);", "a += term;"),
    "first_block_skipped": ("for (int64_t b = 0; b < KB; ++b) {\n                const int32_t S",
                            "for (int64_t b = 1; b < KB; ++b) {\n                const int32_t S"),
    # pos-vector RoPE
    "rope_interleaved_pairs": ("const double b = Y[t * row_stride + h * head_dim + i + half];",
                               "const double b = Y[t * row_stride + h * head_dim + (2 * i + 1) % head_dim];"),
    "rope_exponent_halved": ("pow(base, -2.0 * (double)i / (double)head_dim)",
                             "pow(base, -(double)i / (double)head_dim)"),
    "rope_sign": ("o[i] = a * c - b * sn;", "o[i] = a * c + b * sn;"),
    "rope_first_row_position": ("(double)pos[t] * pow(", "(double)pos[0] * pow("),
    "rope_position_off_by_one": ("(double)pos[t] * pow(", "(double)(pos[t] + 1) * pow("),
    "block_dots_wrong_row": ("? 0\n                             : block_dot(qw + n * K",
                             "? 0\n                             : block_dot(qw + (n ? n - 1 : n) * K"),
}


def _make_mutant(tmp_path, name, old, new):
    src = open(oracle.SOURCE).read()
    assert src.count(old) == 1, f"mutant {name}: pattern must occur exactly once"
    path = tmp_path / f"{name}.c"
    path.write_text(src.replace(old, new))
    lib = str(tmp_path / f"lib{name}.so")
    oracle.compile_oracle(str(path), lib)
    return oracle.Oracle(lib)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    orc = _make_mutant(tmp_path, name, old, new)
    caught = []
    for pin in pins.FAST_PINS:
        try:
            pin(orc)
        except Exception as e:  # noqa: BLE001 - any failure counts as caught
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"no pin detects the planted mistake '{name}'"


def test_unmutated_source_passes(tmp_path):
    """The same build path with no mutation passes every pin."""
    lib = str(tmp_path / "libclean.so")
    oracle.compile_oracle(oracle.SOURCE, lib)
    orc = oracle.Oracle(lib)
    for pin in pins.FAST_PINS:
        pin(orc)


def test_mutant_patterns_exist():
    src = open(oracle.SOURCE).read()
    for name, (old, _) in MUTANTS.items():
        assert src.count(old) == 1, name
    assert os.path.exists(oracle.SOURCE)
