"""Pins for the oracle's binary16 codec and its leaky ReLU, against independent routines.

- binary16 -> binary32 widening: all 65,536 patterns against numpy's own float16 -> float32 cast.
- binary32 -> binary16 rounding: all 2^32 binary32 patterns against numpy's float32 -> float16
  cast (a correctly rounded, round-to-nearest-even library routine).
- leaky ReLU: all binary16 values against its closed form (x >= 0 -> x; x < 0 -> x * half(0.01)
  with a single rounding, computed exactly in float64 and rounded once by numpy), following
  "Profiling neural material inference", section "Bad versus good activation".
"""
import threading

import numpy as np
import pytest

from conftest import host_threads

SLOPE = 0.01000213623046875  # half(0.01) = 0x211f = 1311 * 2^-17, exact in float64


def test_slope_constant_is_half_of_0_01():
    assert np.float16(0.01).view(np.uint16) == 0x211F
    assert float(np.float16(0.01)) == SLOPE == 1311 * 2.0**-17


def test_f16_to_f32_all_patterns(oracle_mod):
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = oracle_mod.f16_bits_to_f32(h)
    ref = h.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))  # bit-exact, keeps -0


def test_f32_to_f16_special_values(oracle_mod):
    cases = [
        (0.0, 0x0000), (-0.0, 0x8000), (1.0, 0x3C00), (-2.0, 0xC000), (65504.0, 0x7BFF),
        (65519.99, 0x7BFF), (65520.0, 0x7C00), (1e9, 0x7C00), (-1e9, 0xFC00),
        (2.0**-14, 0x0400), (2.0**-24, 0x0001), (2.0**-25, 0x0000), (3 * 2.0**-26, 0x0001),
        (float("inf"), 0x7C00), (float("-inf"), 0xFC00),
        (1.0 + 2.0**-11, 0x3C00),            # tie -> even (down)
        (1.0 + 3 * 2.0**-11, 0x3C02),        # tie -> even (up)
        (0.01, 0x211F),
    ]
    got = oracle_mod.f32_to_f16_bits(np.array([v for v, _ in cases], dtype=np.float32))
    assert [hex(int(g)) for g in got] == [hex(b) for _, b in cases]
    assert int(oracle_mod.f32_to_f16_bits(np.array([np.nan], np.float32))[0]) & 0x7FFF > 0x7C00


def test_f32_to_f16_exhaustive_against_numpy(oracle_mod):
    """Every one of the 2^32 binary32 bit patterns rounds to the same binary16 as numpy's cast."""
    chunk = 1 << 22
    n_chunks = (1 << 32) // chunk
    bad = []
    lock = threading.Lock()
    next_chunk = [0]

    def worker():
        while True:
            with lock:
                c = next_chunk[0]
                next_chunk[0] += 1
            if c >= n_chunks:
                return
            bits = np.arange(chunk, dtype=np.uint32) + np.uint32(c * chunk)
            x = bits.view(np.float32)
            got = oracle_mod.f32_to_f16_bits(x)
            with np.errstate(over="ignore"):  # values beyond binary16 round to infinity, as intended
                ref = x.astype(np.float16).view(np.uint16)
            isnan = np.isnan(x)
            ok = (got == ref) | (isnan & ((got & 0x7FFF) > 0x7C00))
            if not ok.all():
                i = int(np.flatnonzero(~ok)[0])
                with lock:
                    bad.append((hex(int(bits[i])), hex(int(got[i])), hex(int(ref[i]))))

    ts = [threading.Thread(target=worker) for _ in range(host_threads())]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    assert not bad, bad[:5]


def test_leaky_exhaustive_closed_form(oracle_mod):
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    v = h.view(np.float16).astype(np.float64)
    keep = ~np.isnan(v)
    h, v = h[keep], v[keep]
    assert h.size == 63490  # every non-NaN binary16 value
    got = oracle_mod.leaky_f16_bits(h)
    # x < 0: the float64 product of two binary16 values is exact; numpy rounds it once to binary16.
    ref = np.where(v < 0, (v * SLOPE).astype(np.float16).view(np.uint16), h)
    assert np.array_equal(got, ref)
    # f(x) = x bit-exactly for every x >= 0, and -0 stays -0
    nonneg = (v > 0) | (h == 0x0000)
    assert np.array_equal(got[nonneg], h[nonneg])
    assert int(oracle_mod.leaky_f16_bits(np.array([0x8000], np.uint16))[0]) == 0x8000


def test_leaky_bad_and_good_forms_agree(oracle_mod):
    """The indexed 'if (v < 0) v *= half(0.01)' form and max(v, v*half(0.01)) are the same function
    on every non-NaN binary16 value ("Bad versus good activation")."""
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    v = h.view(np.float16)
    keep = ~np.isnan(v)
    h, v = h[keep], v[keep]
    bad = v.copy()
    neg = bad < 0
    bad[neg] = (bad[neg].astype(np.float64) * SLOPE).astype(np.float16)
    assert np.array_equal(oracle_mod.leaky_f16_bits(h), bad.view(np.uint16))
