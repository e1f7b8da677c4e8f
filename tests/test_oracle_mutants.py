"""The pins are sharp enough: each plausible mistake planted in a copy of
the oracle (built on the CPU into a temporary directory) must fail at least
one pin.  The real oracle source is never modified."""
import os

import pytest

import _pins
import oracle

SRC = open(oracle.SOURCE).read()

MUTANTS = {
    "tie_last_index_wins": (
        "else if (v > best)", "else if (v >= best)"),
    "adaptive_end_floor": (
        "*end = ((o + 1) * X + O - 1) / O;", "*end = ((o + 1) * X) / O;"),
    "adaptive_start_ceil": (
        "*start = (o * X) / O;", "*start = (o * X + O - 1) / O;"),
    "fixed_start_uses_kernel": (
        "*start = o * s;\n        *end = o * s + k;",
        "*start = o * k;\n        *end = o * k + k;"),
    "fixed_out_ceil_mode": (
        "return (X - k) / s + 1;", "return (X - k + s - 1) / s + 1;"),
    "index_h_w_transposed": (
        "idx[o] = (int32_t)best_i;",
        "idx[o] = (int32_t)(((best_i / (H * W)) * W + best_i % W) * H + (best_i / W) % H);"),
    "ex_index_h_w_transposed": (
        "idx[o] = best_i;",
        "idx[o] = best_i < 0 ? -1 : ((best_i / (H * W)) * W + best_i % W) * H + (best_i / W) % H;"),
    "scan_w_before_h": (
        "for (int64_t h = h0; h < h1; ++h)\n"
        "                            for (int64_t w = w0; w < w1; ++w) {",
        "for (int64_t w = w0; w < w1; ++w)\n"
        "                            for (int64_t h = h0; h < h1; ++h) {"),
    "nan_not_propagated": (
        "else if (isnan(v) && !isnan(best))", "else if (0)"),
    "backward_overwrites": (
        "float sum = acc32[t] + g;", "float sum = g;"),
    "backward_wrong_sign": (
        "float sum = acc32[t] + g;", "float sum = acc32[t] - g;"),
    "backward_drops_last_output": (
        "for (int64_t o = 0; o < plane_out; ++o) {\n            int64_t i = idx",
        "for (int64_t o = 0; o < plane_out - 1; ++o) {\n            int64_t i = idx"),
    "backward_drops_last_cell": (
        "if (i < 0 || i >= plane_in)", "if (i < 0 || i >= plane_in - 1)"),
    "accumulator_starts_negative_zero": (
        "acc32[t] = 0.0f;", "acc32[t] = -0.0f;"),
    "f16_round_truncates": (
        "double mant = rint(ldexp(a, 10 - E));", "double mant = floor(ldexp(a, 10 - E));"),
    "f16_subnormal_round_truncates": (
        "double q = rint(ldexp(a, 24));", "double q = floor(ldexp(a, 24));"),
    "bf16_round_truncates": (
        "double mant = rint(ldexp(a, 7 - E));", "double mant = floor(ldexp(a, 7 - E));"),
    "f16_widen_wrong_bias": (
        "ldexp((double)(1024 + m), e - 25)", "ldexp((double)(1024 + m), e - 24)"),
    "bf16_widen_subnormal_scale": (
        "ldexp((double)m, -133)", "ldexp((double)m, -132)"),
    "ex_tap_ignores_dilation": (
        "q = o * s - pad + j * dil;", "q = o * s - pad + j;"),
    "ex_padding_added": (
        "q = o * s - pad + j * dil;", "q = o * s + pad + j * dil;"),
    "ex_right_padding_read": (
        "return (q >= 0 && q < X) ? q : -1;", "return (q >= 0 && q < X + 1) ? q : -1;"),
    "ex_span_ignores_dilation": (
        "int64_t span = (k - 1) * dil + 1;", "int64_t span = k;"),
    "ex_floor_mode_rounds_up": (
        "if (ceil_mode && n * s < room)", "if (n * s < room)"),
    "ex_ceil_keeps_window_in_padding": (
        "if (ceil_mode && (O - 1) * s >= X + pad)", "if (0)"),
    "argmax_from_output_last_match": (
        "for (int64_t jw = 0; jw < nt[2] && found < 0; ++jw) {",
        "for (int64_t jw = 0; jw < nt[2]; ++jw) {"),
    "argmax_from_output_nan_unmatched": (
        "if (isnan(want) ? isnan(v) : v == want)", "if (v == want)"),
    "f64_backward_rounded_to_binary32": (
        "g64[t] = g64[t] + gv;", "g64[t] = (float)(g64[t] + gv);"),
    "f64_loaded_as_binary32": (
        "return ((const double *)buf)[i];", "return (float)((const double *)buf)[i];"),
    "ex_empty_window_zero": (
        "((float *)y)[o] = -INFINITY;", "((float *)y)[o] = 0.0f;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    assert SRC.count(old) == 1, "mutation site not unique: %s" % name
    src = tmp_path / "mutant.c"
    src.write_text(SRC.replace(old, new))
    lib = oracle.build(str(src), str(tmp_path / "libmutant.so"))
    orc = oracle.Oracle(lib)
    for pin in _pins.ALL_PINS:
        try:
            pin(orc)
        except AssertionError:
            return
    pytest.fail("no pin caught mutant %s" % name)
