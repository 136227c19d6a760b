"""Pins for the oracle's qwZ block quantization ("DeepSpeed ZeRO Stages" 5.3;
the ZeRO++ discussion of "ZeRO Optimization: Stages 1, 2, and 3
Explained": fp16 weights sent as INT8 with per-block scales).  Reading:
blocks of 256, scale = max|x|/127, code = clamp(rint(x/scale), +-127).

Pinned by cases with a closed answer -- values that are exact multiples of a
power-of-two scale, exact ties (round half to even), zero blocks, the block
maximum mapping to +-127 -- and the round-trip error bound
|deq(q(x)) - x| <= scale/2 (+ half an fp16 ulp of the result)."""
import numpy as np
import pytest


def _f16(values):
    return np.asarray(values, dtype=np.float16).view(np.uint16)


def test_exact_multiples_of_power_of_two_scale(orc):
    # max|x| = 127 * 2^-10 -> scale = 2^-10 exactly; x = k * 2^-10 -> code k
    k = np.concatenate([np.arange(-127, 128), [127]]).astype(np.int64)       # 256 values
    x = _f16(k * 2.0 ** -10)
    codes, scales = orc.qwz_quantize(x)
    assert scales[0] == np.float32(2.0 ** -10)
    assert np.array_equal(codes.astype(np.int64), k)
    assert np.array_equal(orc.qwz_dequantize(codes, scales), x)


def test_ties_round_half_to_even(orc):
    # scale = 2^-8; x = (k + 1/2) * 2^-8 are exact ties
    k = np.arange(-20, 20)
    x = np.concatenate([[127 * 2.0 ** -8], (k + 0.5) * 2.0 ** -8])
    codes, _ = orc.qwz_quantize(_f16(x))
    want = np.round(k + 0.5)           # numpy rounds half to even
    assert np.array_equal(codes[1:].astype(np.int64), want.astype(np.int64))
    assert codes[0] == 127


def test_zero_block_and_extremes(orc):
    x = np.zeros(300, dtype=np.float16)
    x[256 + 7] = -3.5                   # second (partial) block: max |x| at a negative value
    x[256 + 9] = 1.0
    codes, scales = orc.qwz_quantize(x.view(np.uint16))
    assert scales.size == 2 and scales[0] == 0.0 and not codes[:256].any()
    assert codes[256 + 7] == -127
    assert scales[1] == np.float32(np.float32(3.5) / np.float32(127.0))


@pytest.mark.parametrize("sigma", [0.02, 3.0, 1e-5])
def test_round_trip_error_bound(orc, sigma):
    rng = np.random.default_rng(int(sigma * 1e6) + 1)
    x = _f16(rng.standard_normal(256 * 40 + 77) * sigma)
    codes, scales = orc.qwz_quantize(x)
    back = orc.qwz_dequantize(codes, scales).view(np.float16).astype(np.float64)
    xf = x.view(np.float16).astype(np.float64)
    sc = np.repeat(scales.astype(np.float64), 256)[: x.size]
    half_ulp = np.spacing(np.abs(back).astype(np.float16)).astype(np.float64) / 2
    assert (np.abs(back - xf) <= sc / 2 * (1 + 2.0 ** -20) + half_ulp + 1e-30).all()
    assert (np.abs(codes.astype(np.int64)) <= 127).all()
    # the element holding each block's maximum maps to +-127
    for b in range(scales.size):
        blk = np.abs(xf[b * 256:(b + 1) * 256])
        if blk.max() > 0:
            assert np.abs(codes[b * 256 + int(np.argmax(blk))]) == 127


def test_decode_of_encoder_scales_is_the_once_rounded_product(orc):
    """Decoding forms code * scale in binary32 and then rounds to fp16. For
    every scale the encoder can produce (max|x|/127 of an fp16 block), that
    equals the exact product rounded once to fp16. The check is exhaustive
    over all positive finite fp16 maxima and all codes. The exact product
    (at most 32 significant bits) is exact in double, and numpy narrows a
    double to fp16 with a single rounding."""
    maxima = np.arange(1, 0x7C00, dtype=np.uint16)          # every positive finite fp16
    x = np.zeros((maxima.size, 256), dtype=np.uint16)
    x[:, 0] = maxima
    _, scales = orc.qwz_quantize(x.reshape(-1))
    assert scales.size == maxima.size
    codes = np.zeros((maxima.size, 256), dtype=np.int8)
    codes[:, :255] = np.arange(-127, 128, dtype=np.int8)
    got = orc.qwz_dequantize(codes.reshape(-1), scales).reshape(maxima.size, 256)
    exact = codes.astype(np.float64) * scales.astype(np.float64)[:, None]
    assert np.array_equal(got, exact.astype(np.float16).view(np.uint16))
    # the two roundings do differ for scales the encoder never produces
    c = np.arange(-127, 128, dtype=np.float64)
    other = np.random.default_rng(3).uniform(1e-4, 1.0, 4000).astype(np.float32)
    ex = c[None, :] * other.astype(np.float64)[:, None]
    assert (ex.astype(np.float16).view(np.uint16) != ex.astype(np.float32).astype(np.float16).view(np.uint16)).any()
