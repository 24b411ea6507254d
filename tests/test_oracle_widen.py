"""Pins for oracle.widen, the only arithmetic-free step between stored inputs and the oracle: a bf16
element is the top half of an IEEE binary32 pattern (sign, 8 exponent bits, 7 stored fraction bits),
so its value is fixed by that definition and is written out below independently of any float type.
Also pins the input generator's float32 -> bf16 rounding (nearest, ties to even)."""
import math

import numpy as np

import oracle
from head_attention_flash_amd import synth


def _bf16_value(bits: int) -> float:
    """Value of a bf16 bit pattern from the IEEE binary32 definition (exponent bias 127)."""
    sign = -1.0 if bits & 0x8000 else 1.0
    exp = (bits >> 7) & 0xFF
    frac = bits & 0x7F
    if exp == 0xFF:
        return sign * math.inf if frac == 0 else math.nan
    if exp == 0:
        return sign * math.ldexp(frac, -126 - 7)   # subnormal: 0.frac x 2^-126
    return sign * math.ldexp(128 + frac, exp - 127 - 7)


CASES = {
    0x3F80: 1.0, 0xBF80: -1.0, 0x4000: 2.0, 0xC000: -2.0, 0x3FC0: 1.5, 0x3F81: 1.0 + 2.0 ** -7,
    0x7F7F: (2.0 - 2.0 ** -7) * 2.0 ** 127,          # largest finite
    0x0080: 2.0 ** -126,                            # smallest normal
    0x0001: 2.0 ** -133,                            # smallest subnormal
    0x007F: 127 * 2.0 ** -133,                      # largest subnormal
    0x0000: 0.0, 0x8000: -0.0, 0x4049: 3.140625, 0xC2F7: -123.5,
    0x7F80: math.inf, 0xFF80: -math.inf,
}


def test_widen_fixed_bf16_patterns():
    bits = np.array(list(CASES), dtype=np.uint16)
    got = oracle.widen(bits)
    assert got.dtype == np.float64
    for b, g in zip(CASES, got):
        want = CASES[b]
        assert g == want and math.copysign(1.0, g) == math.copysign(1.0, want), (hex(b), g, want)
        assert _bf16_value(b) == want, hex(b)


def test_widen_every_bf16_pattern_matches_the_definition():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    with np.errstate(invalid="ignore"):  # NaN patterns widen to NaN
        got = oracle.widen(bits)
    want = np.array([_bf16_value(int(b)) for b in bits])
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))  # -0.0 stays negative


def test_widen_float32_is_exact():
    x = np.array([1.0, -0.1, 3.4028234663852886e38, 1.401298464324817e-45, 0.0], dtype=np.float32)
    got = oracle.widen(x)
    assert got.dtype == np.float64
    assert [float(v) for v in got] == [float(v) for v in x.tolist()]


def test_input_rounding_is_nearest_even():
    # float32 bit patterns and their bf16 rounding: below, at and above the halfway point
    f = np.array([0x3F808000, 0x3F818000, 0x3F808001, 0x3F807FFF, 0xBF808000, 0x7F7FFFFF, 0x00008000],
                 dtype=np.uint32).view(np.float32)
    want = [0x3F80, 0x3F82, 0x3F81, 0x3F80, 0xBF80, 0x7F80, 0x0000]
    assert synth.f32_to_bf16_bits(f).tolist() == want
    # the rounded value is the nearest bf16 value (ties to the even fraction)
    r = np.random.default_rng(0).standard_normal(4096).astype(np.float32)
    b = synth.f32_to_bf16_bits(r)
    v = oracle.widen(b)
    up = oracle.widen(b + 1)
    dn = oracle.widen(b - 1)
    x = r.astype(np.float64)
    assert np.all(np.abs(v - x) <= np.minimum(np.abs(up - x), np.abs(dn - x)))
