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
