"""Pins for the oracle's binary16 conversions (IEEE-754 definitions).

The oracle's decode and round-to-nearest-even encode are compared with numpy's
float16 conversion, an independent library routine: decode over all 65,536
codes; encode over every combination of the top 16 bits of a binary32 with
rounding-boundary patterns of the low 16 bits plus random codes (the full
2^32 sweep is the opt-in ``slow`` test).
"""
import numpy as np
import pytest


def _same_f16(a, b, x):
    """Bitwise equality, NaNs compared as a class (payloads may differ)."""
    nan_in = np.isnan(x)
    a_nan = ((a & 0x7C00) == 0x7C00) & ((a & 0x03FF) != 0)
    b_nan = ((b & 0x7C00) == 0x7C00) & ((b & 0x03FF) != 0)
    return np.where(nan_in, a_nan & b_nan, a == b)


def test_decode_exhaustive(orc):
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = orc.f16_to_f32(codes)
    ref = codes.view(np.float16).astype(np.float32)
    same = (got.view(np.uint32) == ref.view(np.uint32)) | (np.isnan(got) & np.isnan(ref))
    assert same.all()
    # signs of NaN and zero are kept
    assert np.signbit(got[0x8000]) and got[0x8000] == 0
    assert np.signbit(got[0xFE00]) and np.isnan(got[0xFE00])


LOW_PATTERNS = np.array([0x0000, 0x0001, 0x0002, 0x0FFF, 0x1000, 0x1001, 0x17FF,
                         0x1800, 0x1FFF, 0x2000, 0x2001, 0x3000, 0x5000, 0x7FFF,
                         0x8000, 0x8001, 0x9000, 0xB000, 0xD000, 0xEFFF, 0xF000,
                         0xF001, 0xFFFE, 0xFFFF], dtype=np.uint32)


def test_encode_stratified(orc):
    rng = np.random.default_rng(0xF16)
    hi = np.arange(65536, dtype=np.uint32) << 16
    lows = np.concatenate([LOW_PATTERNS, rng.integers(0, 65536, 8, dtype=np.uint32)])
    codes = (hi[:, None] | lows[None, :]).ravel()
    codes = np.concatenate([codes, rng.integers(0, 2**32, 4_000_000, dtype=np.uint64).astype(np.uint32)])
    x = codes.view(np.float32)
    got = orc.f32_to_f16(x)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    assert _same_f16(got, ref, x).all()


@pytest.mark.parametrize("value,code", [
    (65504.0, 0x7BFF),             # largest finite
    (65519.996, 0x7BFF),           # just below the overflow tie
    (65520.0, 0x7C00),             # tie between 65504 and 2^16 -> even -> inf
    (-65520.0, 0xFC00),
    (2.0**-24, 0x0001),            # smallest subnormal
    (2.0**-25, 0x0000),            # tie between 0 and 2^-24 -> even (0)
    (1.5 * 2.0**-25, 0x0001),
    (3 * 2.0**-25, 0x0002),        # tie between codes 1 and 2 -> even (2)
    (2.0**-14, 0x0400),            # smallest normal
    (2.0**-14 - 2.0**-25, 0x0400), # rounds up into the normal range
    (1.0 + 2.0**-11, 0x3C00),      # tie -> even mantissa
    (1.0 + 3 * 2.0**-11, 0x3C02),  # tie -> even mantissa (up)
    (-0.0, 0x8000),
    (0.02, 0x251F),
])
def test_encode_known_values(orc, value, code):
    assert int(orc.f32_to_f16(np.array([value], dtype=np.float32))[0]) == code


@pytest.mark.slow
def test_encode_exhaustive(orc):
    chunk = 1 << 26
    for start in range(0, 1 << 32, chunk):
        codes = np.arange(start, start + chunk, dtype=np.uint64).astype(np.uint32)
        x = codes.view(np.float32)
        got = orc.f32_to_f16(x)
        with np.errstate(over="ignore"):
            ref = x.astype(np.float16).view(np.uint16)
        assert _same_f16(got, ref, x).all(), hex(start)
