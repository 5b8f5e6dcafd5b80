"""Pins for the CFG combine oracle and its float32 FMA emulation (CPU only)."""

from fractions import Fraction

import numpy as np
import pytest

from oracle import brute, cfg_combine, cfg_combine_f32, fmaf

RNG = np.random.default_rng(5)


def _round_f32(x: Fraction) -> np.float32:
    """Correct round-to-nearest-even of an exact rational to float32 (normal
    range), from the definition: scale to a 24-bit significand and round."""
    if x == 0:
        return np.float32(0.0)
    sign = -1 if x < 0 else 1
    x = abs(x)
    e = x.numerator.bit_length() - x.denominator.bit_length()
    while Fraction(2) ** e > x:
        e -= 1
    while Fraction(2) ** (e + 1) <= x:
        e += 1
    m = x / Fraction(2) ** (e - 23)           # in [2^23, 2^24)
    fl = m.numerator // m.denominator
    rem = m - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return np.float32(sign * float(Fraction(fl) * Fraction(2) ** (e - 23)))


def test_matches_brute_force():
    u = RNG.standard_normal(50)
    c = RNG.standard_normal(50)
    np.testing.assert_allclose(cfg_combine(u, c, 3.7), brute.cfg(u.tolist(), c.tolist(), 3.7),
                               atol=1e-15)


def test_special_guidance_values():
    u = RNG.standard_normal(100).astype(np.float32)
    c = RNG.standard_normal(100).astype(np.float32)
    np.testing.assert_array_equal(cfg_combine(u, c, 0.0), u.astype(np.float64))
    np.testing.assert_allclose(cfg_combine(u, c, 1.0), c.astype(np.float64), atol=1e-15)
    np.testing.assert_array_equal(cfg_combine_f32(u, c, 0.0), u)


def test_f32_path_for_power_of_two_guidance_is_plain_float32():
    # g = 4: 4 * fl32(c - u) is exact, so the fused and the unfused float32
    # evaluations agree bit for bit.
    u = RNG.standard_normal(1000).astype(np.float32)
    c = RNG.standard_normal(1000).astype(np.float32)
    plain = (u + np.float32(4.0) * (c - u)).astype(np.float32)
    np.testing.assert_array_equal(cfg_combine_f32(u, c, 4.0), plain)


def test_f32_path_is_close_to_float64():
    u = RNG.standard_normal(1000).astype(np.float32)
    c = RNG.standard_normal(1000).astype(np.float32)
    for g in (4.0, 7.5, 1.3):
        np.testing.assert_allclose(cfg_combine_f32(u, c, g), cfg_combine(u, c, g), atol=1e-5)


def test_fmaf_is_correctly_rounded_on_random_triples():
    a = RNG.standard_normal(300).astype(np.float32)
    b = RNG.standard_normal(300).astype(np.float32)
    c = RNG.standard_normal(300).astype(np.float32)
    got = fmaf(a, b, c)
    for i in range(300):
        exact = Fraction(float(a[i])) * Fraction(float(b[i])) + Fraction(float(c[i]))
        assert got[i] == _round_f32(exact), i


def test_fmaf_single_rounding_beats_double_rounding_trap():
    # a*b = 2^-24 + k*2^-70 with 0 < k < 2^17: the exact 1 + a*b lies just
    # above the float32 midpoint 1 + 2^-24, but rounding to float64 first
    # lands exactly on the midpoint and ties to 1.0.  Find such 24-bit
    # significands x*y = 2^46 + k.
    for x in range(1 << 23, (1 << 23) + 200000):
        y = -(-(1 << 46) // x)
        k = x * y - (1 << 46)
        if y < (1 << 24) and 0 < k < (1 << 17):
            break
    else:
        pytest.fail("no trap operands found")
    a = np.float32(x * 2.0 ** -35)
    b = np.float32(y * 2.0 ** -35)
    one = np.float32(1.0)
    naive = np.float32(np.float64(a) * np.float64(b) + np.float64(one))
    assert naive == one                                   # the trap is real
    assert fmaf(a, b, one) == np.float32(1.0 + 2.0 ** -23)


def test_fmaf_exact_tie_rounds_to_even():
    a = np.float32(1 + 2.0 ** -12)
    c = np.float32(-(2.0 ** -11))
    # (1 + 2^-12)^2 - 2^-11 = 1 + 2^-24: an exact tie, to even -> 1.0
    assert fmaf(a, a, c) == np.float32(1.0)
