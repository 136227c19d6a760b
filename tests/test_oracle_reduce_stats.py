"""Pins for the oracle's owner-side gradient reduce and gradient statistics.

Reduce ("DeepSpeed ZeRO Stages" 3.1-3.2; "DeepSpeed ZeRO: Extreme Memory
Efficiency", communication section: the reduce-scatter sums):
  * integer-valued fp16 inputs have an exact fp32 sum equal to the integer sum;
  * N = 1 is the identity on all 65,536 codes;
  * random inputs stay within the textbook bound |fl(S) - S| <= (N-1) u sum|x|
    against the exact sum (a sum of <= 64 binary16 values is exact in double);
  * a hand-worked case where the order matters fixes the left fold in rank
    order (reading of "reduction-order effects", section 2 of the first page).
Stats ("DeepSpeed ZeRO Stages" 2.1: clipping needs the global 2-norm):
  * the overflow flag is the OR over injected inf/NaN positions;
  * the sum of squares equals the exact rational sum on small inputs.
"""
from fractions import Fraction

import numpy as np
import pytest

U32 = 2.0 ** -24  # unit roundoff of binary32


def _f16(values):
    return np.asarray(values, dtype=np.float16).view(np.uint16)


@pytest.mark.parametrize("n", [1, 2, 3, 4, 7, 16, 33, 64])
def test_reduce_integer_exact(orc, n):
    rng = np.random.default_rng(n)
    ints = rng.integers(-2048, 2049, size=(n, 5000))
    slices = [_f16(row.astype(np.float32)) for row in ints]
    out = orc.grad_reduce(slices)
    assert np.array_equal(out.astype(np.int64), ints.sum(axis=0))


def test_reduce_identity_n1(orc):
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    out = orc.grad_reduce([codes])
    ref = codes.view(np.float16).astype(np.float32)
    assert ((out.view(np.uint32) == ref.view(np.uint32)) | (np.isnan(out) & np.isnan(ref))).all()


@pytest.mark.parametrize("n,scale", [(2, 1.0), (4, 65.536), (8, 1e-3), (64, 4.096), (64, 1e4)])
def test_reduce_error_bound(orc, n, scale):
    rng = np.random.default_rng(100 + n)
    vals = (rng.standard_normal((n, 20000)) * scale).astype(np.float16)
    out = orc.grad_reduce([row.view(np.uint16) for row in vals])
    exact = vals.astype(np.float64).sum(axis=0)        # exact: <= 64 binary16 terms
    bound = (n - 1) * U32 * np.abs(vals.astype(np.float64)).sum(axis=0)
    assert (np.abs(out.astype(np.float64) - exact) <= bound).all()


def test_reduce_order_is_left_fold_in_rank_order(orc):
    # binary32 with ties to even: 1 + 2^-24 rounds back to 1, but
    # 2^-24 + 2^-24 = 2^-23 is exact and 2^-23 + 1 is representable.
    tiny = 2.0 ** -24
    a = orc.grad_reduce([_f16([1.0]), _f16([tiny]), _f16([tiny])])
    b = orc.grad_reduce([_f16([tiny]), _f16([tiny]), _f16([1.0])])
    assert a[0] == np.float32(1.0)
    assert b[0] == np.float32(1.0 + 2.0 ** -23)


def test_reduce_signed_zero_and_specials(orc):
    nz = _f16([-0.0])
    assert np.signbit(orc.grad_reduce([nz, nz, nz])[0])            # -0 + -0 = -0
    assert not np.signbit(orc.grad_reduce([nz, _f16([0.0])])[0])   # -0 + +0 = +0
    inf, ninf, nan = _f16([np.inf]), _f16([-np.inf]), _f16([np.nan])
    assert orc.grad_reduce([_f16([1.0]), inf])[0] == np.inf
    assert np.isnan(orc.grad_reduce([inf, ninf])[0])
    assert np.isnan(orc.grad_reduce([nan, _f16([2.0])])[0])
    # the largest possible finite sum stays finite: 64 * 65504 < FLT_MAX
    big = orc.grad_reduce([_f16([65504.0])] * 64)[0]
    assert big == np.float32(64 * 65504.0)


def test_stats_flag_counts_injected(orc):
    rng = np.random.default_rng(7)
    g = _f16(rng.standard_normal(100000) * 60)
    assert orc.grad_stats(g, 2.0 ** -16)[0] == 0
    for special in (np.inf, -np.inf, np.nan):
        for pos in (0, 12345, 99999):
            h = g.copy()
            h[pos] = _f16([special])[0]
            assert orc.grad_stats(h, 2.0 ** -16)[0] == 1
    g32 = rng.standard_normal(1000).astype(np.float32)
    assert orc.grad_stats(g32, 1.0)[0] == 0
    g32[500] = np.inf
    assert orc.grad_stats(g32, 1.0)[0] == 1


@pytest.mark.parametrize("scale_pow", [-16, -18, 0])
def test_stats_sumsq_exact_rational(orc, scale_pow):
    rng = np.random.default_rng(11 - scale_pow)
    x = (rng.standard_normal(3000) * 64).astype(np.float16)
    s = 2.0 ** scale_pow
    _, ssq = orc.grad_stats(x.view(np.uint16), s)
    # g = x * s is exact (power-of-two scale, no underflow), so the exact value
    # is the rational sum of (x*s)^2
    exact = sum(Fraction(float(v)) ** 2 for v in x.astype(np.float64)) * Fraction(s) ** 2
    assert abs(Fraction(ssq) - exact) <= exact * Fraction(1, 2**50)


def test_stats_sumsq_f32_exact_rational(orc):
    rng = np.random.default_rng(5)
    x = (rng.standard_normal(2000) * 100).astype(np.float32)
    s = 2.0 ** -18
    _, ssq = orc.grad_stats(x, s)
    exact = sum((Fraction(float(v)) * Fraction(s)) ** 2 for v in x)
    assert abs(Fraction(ssq) - exact) <= exact * Fraction(1, 2**50)


def test_stats_zero_and_empty(orc):
    assert orc.grad_stats(np.zeros(10, np.uint16), 2.0 ** -16) == (0, 0.0)
    assert orc.grad_stats(np.zeros(0, np.uint16), 2.0 ** -16) == (0, 0.0)
