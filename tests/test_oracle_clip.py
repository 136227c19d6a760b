"""Pins for the oracle's global-norm gradient clipping ("DeepSpeed ZeRO
Stages" 2.1: clipping needs the 2-norm over all of P).  Reading: with
norm = sqrt(sum of squares of the unscaled gradient), the gradient is scaled
by max_norm / norm when norm > max_norm; the factor is folded into the
unscale multiplier (one rounding).

Pinned by the defining property -- the clipped gradient's 2-norm is max_norm,
checked in exact rational arithmetic within the binary32 rounding of each
element -- by the no-op cases, and by the t = 1 closed form with clipping."""
from fractions import Fraction

import numpy as np
import pytest

LR, B1, B2, EPS = 1e-4, 0.9, 0.999, 1e-8
U = 2.0 ** -24


def _f16(values):
    return np.asarray(values, dtype=np.float16).view(np.uint16)


def test_factor_no_op_cases(orc):
    assert orc.clip_factor(4.0, 0.0) == 1.0          # clipping off
    assert orc.clip_factor(4.0, -1.0) == 1.0
    assert orc.clip_factor(0.0, 1.0) == 1.0          # zero gradient
    assert orc.clip_factor(4.0, 2.0) == 1.0          # norm == bound: untouched
    assert orc.clip_factor(3.99, 2.0) == 1.0         # below the bound
    assert orc.clip_factor(16.0, 2.0) == 0.5         # norm 4 -> factor 2/4


@pytest.mark.parametrize("max_norm", [1e-3, 0.01, 0.05])
def test_clipped_norm_equals_bound(orc, max_norm):
    rng = np.random.default_rng(int(max_norm * 1e6))
    x16 = _f16(rng.standard_normal(4000) * 1e-3 * 65536)
    s = 2.0 ** -16
    flag, ssq = orc.grad_stats(x16, s)
    assert flag == 0
    norm = float(np.sqrt(ssq))
    assert norm > max_norm                       # the bound is active
    factor = orc.clip_factor(ssq, max_norm)
    s_eff = np.float32(s * factor)
    g = x16.view(np.float16).astype(np.float32) * s_eff          # binary32 products
    clipped = sum(Fraction(float(v)) ** 2 for v in g)
    # each element carries at most two binary32 roundings (s_eff, product)
    rel = Fraction(4 * U)
    assert abs(clipped - Fraction(max_norm) ** 2) <= rel * Fraction(max_norm) ** 2


def test_step_with_clipping_t1_closed_form(orc):
    rng = np.random.default_rng(77)
    n = 20000
    th0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    x16 = _f16(rng.standard_normal(n) * 1e-3 * 65536)
    s = 2.0 ** -16
    max_norm = 0.01
    th, m, v = th0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    p = np.zeros(n, np.uint16)
    st, flag, ssq = orc.shard_adam_step(x16, th, m, v, p, step=1, lr=LR, beta1=B1, beta2=B2, eps=EPS,
                                        inv_scale=s, max_norm=max_norm)
    assert st == 0 and flag == 0
    assert np.sqrt(ssq) > max_norm
    # m' = (1-b1) g_c with ||g_c|| = max_norm
    gc = m.astype(np.float64) / 0.1
    assert abs(np.sqrt((gc ** 2).sum()) - max_norm) <= 8 * U * max_norm
    # t = 1: theta' = theta - lr * g_c/(|g_c| + eps) with g_c = f32(x) * max_norm/norm * s
    g = x16.view(np.float16).astype(np.float64) * s * (max_norm / np.sqrt(ssq))
    u = g / (np.abs(g) + EPS)
    closed = th0.astype(np.float64) - LR * u
    ulp = np.spacing(np.abs(th)).astype(np.float64)
    assert (np.abs(th - closed) <= ulp / 2 + 12 * U * LR * np.abs(u)).all()
    # without clipping the result differs (the bound is active): v is g^2-scaled
    th2, m2, v2 = th0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    orc.shard_adam_step(x16, th2, m2, v2, p.copy(), step=1, lr=LR, beta1=B1, beta2=B2, eps=EPS, inv_scale=s)
    assert not np.array_equal(v, v2)


def test_clipping_inactive_is_bit_identical(orc):
    rng = np.random.default_rng(78)
    n = 5000
    th0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m0 = (rng.standard_normal(n) * 1e-4).astype(np.float32)
    v0 = np.abs(rng.standard_normal(n) * 1e-6).astype(np.float32)
    x16 = _f16(rng.standard_normal(n) * 65.536)
    outs = []
    for mn in (0.0, 1e6):
        a = [th0.copy(), m0.copy(), v0.copy(), np.zeros(n, np.uint16)]
        st, flag, _ = orc.shard_adam_step(x16, *a, step=9, lr=LR, beta1=B1, beta2=B2, eps=EPS,
                                          inv_scale=2.0 ** -16, max_norm=mn)
        assert st == 0 and flag == 0
        outs.append(a)
    for x, y in zip(*outs):
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8))


def test_invalid_max_norm(orc):
    a = [np.zeros(4, np.float32), np.zeros(4, np.float32), np.zeros(4, np.float32), np.zeros(4, np.uint16)]
    st, _, _ = orc.shard_adam_step(np.zeros(4, np.uint16), *a, step=1, lr=LR, beta1=B1, beta2=B2, eps=EPS,
                                   inv_scale=1.0, max_norm=float("nan"))
    assert st == -1
