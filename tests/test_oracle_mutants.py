"""The pins discriminate: each planted mistake in a copy of the oracle's C source fails one of them.

The mistakes are planted on the CPU only, in temporary copies built with the same gcc flags; the
real ``oracle/mlp_oracle.c`` is untouched.  Every mutant below is a plausible slip in writing the
oracle (a dropped term or bias, a wrong index or orientation, a wrong activation, slope, rounding
mode or accumulation precision, a codec off by one), and the quick pins must reject every one.
"""
import shutil

import numpy as np
import pytest

import test_oracle_codec as codec
import test_oracle_fp8 as fp8
import test_oracle_pins as pins
from oracle import oracle as oracle_pkg

MUTANTS = {
    "dropped_bias": ("float acc = oracle_f16_to_f32(b[j]);", "float acc = 0.0f;"),
    "dropped_last_term": ("for (int i = 0; i < w_in; ++i)", "for (int i = 0; i + 1 < w_in; ++i)"),
    "reversed_input_index": ("* oracle_f16_to_f32(h[i]);", "* oracle_f16_to_f32(h[w_in - 1 - i]);"),
    "transposed_weights": ("W[(size_t)j * w_in + i]", "W[(size_t)(i % w_out) * w_in + (j % w_in)]"),
    "relu_not_leaky": ("return (fs > fv) ? scaled : v;", "return (fv > 0.0f) ? v : (uint16_t)0;"),
    "min_not_max": ("return (fs > fv) ? scaled : v;", "return (fs < fv) ? scaled : v;"),
    "activation_after_output": ("if (l + 1 < n_layers)", "if (l < n_layers)"),
    "slope_1_over_128": ("#define ORACLE_SLOPE_BITS 0x211fu", "#define ORACLE_SLOPE_BITS 0x2000u"),
    "round_toward_zero": ("const double r = rint(a / ldexp(1.0, e - 10));",
                          "const double r = trunc(a / ldexp(1.0, e - 10));"),
    "flush_subnormals": ("return sign | (uint16_t)r;", "return sign | (uint16_t)(r >= 1024 ? r : 0);"),
    "subnormal_decode_scale": ("mag = ldexpf((float)f, -24);", "mag = ldexpf((float)f, -25);"),
    "exponent_bias": ("mag = ldexpf((float)(1024 + f), e - 25);", "mag = ldexpf((float)(1024 + f), e - 24);"),
    "fp16_running_sum": (
        "acc = acc + oracle_f16_to_f32(W[(size_t)j * w_in + i]) * oracle_f16_to_f32(h[i]);",
        "acc = oracle_f16_to_f32(oracle_f32_to_f16(acc + oracle_f16_to_f32(W[(size_t)j * w_in + i]) * oracle_f16_to_f32(h[i])));"),
}


# Planted mistakes in the FP8 variant; each must fail one of the FP8 pins.
FP8_MUTANTS = {
    "fp8_activation_not_scaled": ("oracle_f32_to_e4m3(16.0f * oracle_f16_to_f32(h[k]))",
                                  "oracle_f32_to_e4m3(oracle_f16_to_f32(h[k]))"),
    "fp8_activation_not_quantised": (
        "xq[k] = ldexpf(oracle_e4m3_to_f32(oracle_f32_to_e4m3(16.0f * oracle_f16_to_f32(h[k]))), -4);",
        "xq[k] = oracle_f16_to_f32(h[k]);"),
    "fp8_weight_not_quantised": ("wq[l][(size_t)r * win + k] = ldexpf(oracle_e4m3_to_f32(q), E);",
                                 "wq[l][(size_t)r * win + k] = oracle_f16_to_f32(row[k]) + 0.0f * q;"),
    "fp8_row_exponent_mx_floor": ("while (amax > ldexp(448.0, E))", "while (amax >= ldexp(512.0, E))"),
    "fp8_truncating_encoder": ("const double r = rint(a / ldexp(1.0, e - 3));",
                               "const double r = trunc(a / ldexp(1.0, e - 3));"),
    "fp8_saturating_encoder": ("if (a > 464.0)\n        return sign | 0x7f;", "if (a > 464.0)\n        return sign | 0x7e;"),
    "fp8_subnormal_scale": ("mag = ldexpf((float)f, -9);", "mag = ldexpf((float)f, -10);"),
    # the FP8 network's own activation call and the sign of its encoder
    "fp8_relu_not_leaky": ("                    v = oracle_leaky_f16(v);",
                           "                    v = (v & 0x8000u) ? (uint16_t)0 : v;"),
    "fp8_encoder_drops_sign": ("const uint8_t sign = signbit(x) ? 0x80 : 0;", "const uint8_t sign = 0;"),
}


def _quick_pins_fp8(o):
    yield lambda: fp8.test_encoder_matches_torch_on_binary16_values(o)
    yield lambda: fp8.test_decoder_matches_torch(o)
    yield lambda: fp8.test_row_exponent_keeps_the_row_in_range(o)
    import json

    for case in json.loads(fp8.GOLDEN.read_text())["cases"]:
        yield lambda case=case: fp8.test_hand_worked_examples(o, case)
    for seed in range(3):
        yield lambda seed=seed: fp8.test_integer_exact_nets_match_int64_brute_force(o, seed)
    yield lambda: fp8.test_sign_alternating_diagonal_net_fp8(o)
    yield lambda: fp8.test_fp8_network_is_close_to_the_fp16_network(o, "page")


def _quick_pins(o):
    yield lambda: pins.test_hand_worked_two_layer_net(o)
    yield lambda: pins.test_sign_alternating_diagonal_net(o)
    for w in (4, 32):
        yield lambda w=w: pins.test_identity_passthrough(o, w)
    for widths in [(16, 32, 32, 32, 32, 32, 32, 32, 4), (5, 7, 3, 9)]:
        yield lambda widths=widths: pins.test_all_positive_net_is_one_affine_map(o, widths)
    for seed in range(6):
        yield lambda seed=seed: pins.test_integer_exact_nets_match_int64_brute_force(o, seed)
    yield lambda: pins.test_zero_last_layer_gives_its_bias(o)
    yield lambda: pins.test_zeroed_output_row_gives_exact_zero(o)
    yield lambda: pins.test_accumulation_is_binary32(o)
    yield lambda: codec.test_f16_to_f32_all_patterns(o)
    yield lambda: codec.test_f32_to_f16_special_values(o)
    yield lambda: codec.test_leaky_exhaustive_closed_form(o)


def test_real_oracle_passes_the_quick_pins(oracle_mod):
    for pin in _quick_pins(oracle_mod):
        pin()
    for pin in _quick_pins_fp8(oracle_mod):
        pin()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    src = (oracle_pkg._SRC).read_text()
    assert src.count(old) >= 1, "mutation anchor not found: " + old
    mutant_src = tmp_path / "mutant.c"
    mutant_src.write_text(src.replace(old, new))
    lib = oracle_pkg.build(force=True, src=mutant_src, out=tmp_path / "libmutant.so")
    o = oracle_pkg.Oracle(lib)
    caught = []
    for pin in _quick_pins(o):
        try:
            pin()
        except (AssertionError, ValueError, RuntimeError) as e:
            caught.append(type(e).__name__)
            break
    assert caught, "mutant %r passed every pin" % name


@pytest.mark.parametrize("name", sorted(FP8_MUTANTS))
def test_fp8_mutant_is_caught(tmp_path, name):
    old, new = FP8_MUTANTS[name]
    old, new = old.replace("\\n", "\n"), new.replace("\\n", "\n")
    src = (oracle_pkg._SRC).read_text()
    assert src.count(old) == 1, "mutation anchor not found exactly once: " + old
    mutant_src = tmp_path / "mutant.c"
    mutant_src.write_text(src.replace(old, new))
    lib = oracle_pkg.build(force=True, src=mutant_src, out=tmp_path / "libmutant.so")
    o = oracle_pkg.Oracle(lib)
    caught = []
    for pin in _quick_pins_fp8(o):
        try:
            pin()
        except (AssertionError, ValueError, RuntimeError) as e:
            caught.append(type(e).__name__)
            break
    assert caught, "mutant %r passed every FP8 pin" % name
