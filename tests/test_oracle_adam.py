"""Pins for the oracle's Adam step on a shard.

The update is the one of "DeepSpeed ZeRO Stages" 2.1 (Fact 1) and "ZeRO Stage
1 Math" ("Where the 12 bytes come from"), with bias correction as in Kingma &
Ba (cited by the first page): mhat = m/(1-b1^t), vhat = v/(1-b2^t).

What pins it, independent of how the oracle evaluates it:
  * t = 1 from m = v = 0: mhat = g and vhat = g^2 exactly, so the step is the
    closed form theta - lr*g/(|g|+eps);
  * a constant gradient from m = v = 0: m_k = (1-b1^k) g, v_k = (1-b2^k) g^2
    and theta_k = theta_0 - k*lr*g/(|g|+eps) (geometric series);
  * a zero gradient: m_k = b1^k m_0 and v_k = b2^k v_0;
  * 50-digit decimal evaluation of the real-number update, with a rounding
    bound derived for binary32;
  * invariants: separability (Fact 1: shard-wise == whole), the skip on
    overflow, loss-scale invariance, p16 == f16(master).
"""
from decimal import Decimal, getcontext

import numpy as np
import pytest

U = 2.0 ** -24
LR, B1, B2, EPS = 1e-4, 0.9, 0.999, 1e-8
S16 = 2.0 ** -16


def _f16(values):
    return np.asarray(values, dtype=np.float16).view(np.uint16)


def _ulp32(x):
    return np.spacing(np.abs(np.asarray(x, dtype=np.float32))).astype(np.float64)


def _apply(orc, x16, th, m, v, step, lr=LR, b1=B1, b2=B2, eps=EPS, s=S16, overflow=0):
    th = np.array(th, dtype=np.float32, copy=True)
    m = np.array(m, dtype=np.float32, copy=True)
    v = np.array(v, dtype=np.float32, copy=True)
    p = np.zeros(th.shape, dtype=np.uint16)
    st = orc.adam_apply(x16, th, m, v, p, step=step, lr=lr, beta1=b1, beta2=b2,
                        eps=eps, inv_scale=s, overflow=overflow)
    assert st == 0
    return th, m, v, p


def test_scalars_derived_in_double(orc):
    st, s = orc.adam_scalars(LR, B1, B2, EPS, S16, 1)
    assert st == 0
    # 1-b computed in double then rounded once (not 1.0f - 0.9f)
    assert s[1] == np.float32(0.1) and s[1] != np.float32(1.0) - np.float32(0.9)
    assert s[3] == np.float32(0.001)
    assert s[4] == np.float32(0.1) and s[5] == np.float32(0.001)   # t = 1
    assert s[8] == np.float32(S16)
    _, s10 = orc.adam_scalars(LR, B1, B2, EPS, S16, 10)
    assert s10[4] == np.float32(1 - 0.9 ** 10) and s10[5] == np.float32(1 - 0.999 ** 10)
    _, s1k = orc.adam_scalars(LR, B1, B2, EPS, S16, 1000)
    assert s1k[4] == np.float32(1.0) and s1k[5] == np.float32(1 - 0.999 ** 1000)


@pytest.mark.parametrize("bad", [
    dict(step=0), dict(lr=-1.0), dict(beta1=1.0), dict(beta2=-0.1), dict(eps=0.0),
    dict(inv_scale=0.0), dict(inv_scale=float("inf")), dict(lr=float("nan")),
])
def test_invalid_hyperparameters(orc, bad):
    kw = dict(lr=LR, beta1=B1, beta2=B2, eps=EPS, inv_scale=S16, step=1)
    kw.update(bad)
    st, _ = orc.adam_scalars(kw["lr"], kw["beta1"], kw["beta2"], kw["eps"], kw["inv_scale"], kw["step"])
    assert st == -1


def test_t1_closed_form(orc):
    rng = np.random.default_rng(1)
    n = 200_000
    th0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    x16 = _f16(rng.standard_normal(n) * 1e-3 * 65536)
    zeros = np.zeros(n, np.float32)
    th, m, v, p = _apply(orc, x16, th0, zeros, zeros, 1)
    g = x16.view(np.float16).astype(np.float64) * S16          # exact
    u = g / (np.abs(g) + EPS)
    closed = th0.astype(np.float64) - LR * u
    assert (np.abs(th - closed) <= _ulp32(th) / 2 + 8 * U * LR * np.abs(u)).all()
    assert (np.abs(m - 0.1 * g) <= 3 * U * np.abs(0.1 * g)).all()
    assert (np.abs(v - 0.001 * g * g) <= 4 * U * 0.001 * g * g).all()
    assert np.array_equal(p, orc.f32_to_f16(th))


def test_t1_zero_gradient_is_identity(orc):
    th0 = np.array([0.5, -0.25, 3.0, 0.0], np.float32)
    z = np.zeros(4, np.float32)
    th, m, v, _ = _apply(orc, np.zeros(4, np.uint16), th0, z, z, 1)
    assert np.array_equal(th.view(np.uint32), th0.view(np.uint32))
    assert not m.any() and not v.any()


@pytest.mark.parametrize("k,b1,b2", [(2, 0.9, 0.999), (3, 0.9, 0.999), (10, 0.9, 0.999),
                                     (50, 0.8, 0.99), (7, 0.5, 0.95)])
def test_constant_gradient_closed_form(orc, k, b1, b2):
    rng = np.random.default_rng(k)
    n = 20_000
    th0 = (rng.standard_normal(n) * 0.02 + 0.5).astype(np.float32)
    x16 = _f16(rng.standard_normal(n) * 1e-3 * 65536)
    th, m, v = th0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    for t in range(1, k + 1):
        th, m, v, _ = _apply(orc, x16, th, m, v, t, b1=b1, b2=b2)
    g = x16.view(np.float16).astype(np.float64) * S16
    m_cf = (1 - b1 ** k) * g
    v_cf = (1 - b2 ** k) * g * g
    u = g / (np.abs(g) + EPS)
    th_cf = th0.astype(np.float64) - k * LR * u
    assert (np.abs(m - m_cf) <= (3 * k + 3) * U * np.abs(m_cf)).all()
    assert (np.abs(v - v_cf) <= (3 * k + 4) * U * v_cf).all()
    step_err = LR * np.abs(u) * (8 * k + 12) * U
    # theta moves monotonically, so the largest ulp on its path is at an end
    ulp = np.maximum(_ulp32(th), _ulp32(th0))
    assert (np.abs(th - th_cf) <= k * (ulp / 2 + step_err) + ulp).all()


def test_zero_gradient_pure_decay(orc):
    rng = np.random.default_rng(3)
    n = 10_000
    m0 = (rng.standard_normal(n) * 1e-4).astype(np.float32)
    v0 = np.abs(rng.standard_normal(n) * 1e-6).astype(np.float32)
    th = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m, v = m0.copy(), v0.copy()
    k = 25
    for t in range(1, k + 1):
        th, m, v, _ = _apply(orc, np.zeros(n, np.uint16), th, m, v, t + 100)
    assert (np.abs(m - B1 ** k * m0.astype(np.float64)) <= (2 * k + 1) * U * B1 ** k * np.abs(m0)).all()
    assert (np.abs(v - B2 ** k * v0.astype(np.float64)) <= (2 * k + 1) * U * B2 ** k * v0).all()


def _decimal_step(x, th, m, v, t, s, lr=LR, b1=B1, b2=B2, eps=EPS):
    """Real-number update at 50 digits with the hyperparameters as decimals."""
    getcontext().prec = 50
    D = Decimal
    g = D(float(x)) * D(s)
    b1d, b2d = D(repr(b1)), D(repr(b2))
    m1 = b1d * D(float(m)) + (1 - b1d) * g
    v1 = b2d * D(float(v)) + (1 - b2d) * g * g
    bc1 = 1 - b1d ** t
    bc2 = 1 - b2d ** t
    mh, vh = m1 / bc1, v1 / bc2
    den = vh.sqrt() + D(repr(eps))
    th1 = D(float(th)) - D(repr(lr)) * (mh / den)
    # magnitude scale of the moment before any cancellation, for the bound
    m_mag = (abs(b1d * D(float(m))) + abs((1 - b1d) * g))
    return th1, m1, v1, m_mag / bc1 / den


@pytest.mark.parametrize("name,x,th,m,v,t", [
    ("E1", 64.0, 0.5, 0.0, 0.0, 1),
    ("E2", 64.0, 0.02, 1e-4, 1e-6, 1000),
    ("E5", -3.0, -0.01, -2e-5, 4e-7, 10),
])
def test_worked_examples_decimal(orc, name, x, th, m, v, t):
    th32, m32, v32 = np.float32(th), np.float32(m), np.float32(v)
    tho, mo, vo, _ = _apply(orc, _f16([x]), [th32], [m32], [v32], t)
    th1, m1, v1, scale = _decimal_step(np.float16(x), th32, m32, v32, t, S16)
    assert abs(Decimal(float(mo[0])) - m1) <= Decimal(4 * U) * abs(m1) + Decimal(1e-45)
    assert abs(Decimal(float(vo[0])) - v1) <= Decimal(4 * U) * abs(v1)
    bound = Decimal(float(_ulp32(tho[0]))) + Decimal(repr(LR)) * scale * Decimal(16 * U)
    assert abs(Decimal(float(tho[0])) - th1) <= bound, (name, tho[0], th1)


def test_random_general_decimal(orc):
    rng = np.random.default_rng(1234)
    n = 1500
    th0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m0 = (rng.standard_normal(n) * 1e-4).astype(np.float32)
    v0 = np.abs(rng.standard_normal(n) * 1e-6).astype(np.float32)
    x16 = _f16(rng.standard_normal(n) * 1e-3 * 65536)
    for t in (1, 2, 10, 1000):
        th, m, v, _ = _apply(orc, x16, th0, m0, v0, t)
        for j in range(0, n, 3):
            th1, m1, v1, scale = _decimal_step(x16[j:j + 1].view(np.float16)[0], th0[j], m0[j], v0[j], t, S16)
            mag = abs(Decimal(repr(B1)) * Decimal(float(m0[j]))) + abs(Decimal(repr(1 - B1))) * abs(
                Decimal(float(x16[j:j + 1].view(np.float16)[0])) * Decimal(S16))
            assert abs(Decimal(float(m[j])) - m1) <= Decimal(4 * U) * mag
            assert abs(Decimal(float(v[j])) - v1) <= Decimal(4 * U) * v1
            bound = Decimal(float(_ulp32(th[j]))) + Decimal(repr(LR)) * scale * Decimal(24 * U)
            assert abs(Decimal(float(th[j])) - th1) <= bound, (t, j)


def test_separability_fact1(orc):
    # "DeepSpeed ZeRO Stages" 2.1 Fact 1: the update over P decomposes into
    # independent updates over the shards; bit-identical here.
    rng = np.random.default_rng(9)
    n = 9999
    th0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m0 = (rng.standard_normal(n) * 1e-4).astype(np.float32)
    v0 = np.abs(rng.standard_normal(n) * 1e-6).astype(np.float32)
    x16 = _f16(rng.standard_normal(n) * 65.536)
    whole = _apply(orc, x16, th0, m0, v0, 7)
    cuts = [0, 1, 1000, 4096, 5003, n]
    parts = [_apply(orc, x16[a:b].copy(), th0[a:b], m0[a:b], v0[a:b], 7) for a, b in zip(cuts[:-1], cuts[1:])]
    for i in range(4):
        joined = np.concatenate([p[i] for p in parts])
        assert np.array_equal(joined.view(np.uint8), whole[i].view(np.uint8))


def test_overflow_skip_leaves_state_untouched(orc):
    rng = np.random.default_rng(10)
    n = 5000
    th = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m = (rng.standard_normal(n) * 1e-4).astype(np.float32)
    v = np.abs(rng.standard_normal(n) * 1e-6).astype(np.float32)
    p = orc.f32_to_f16(th)
    x16 = _f16(rng.standard_normal(n) * 65.536)
    x16[1234] = _f16([np.inf])[0]
    copies = [a.copy() for a in (th, m, v, p)]
    st, flag, _ = orc.shard_adam_step(x16, th, m, v, p, step=5, lr=LR, beta1=B1, beta2=B2,
                                      eps=EPS, inv_scale=S16)
    assert st == 0 and flag == 1
    for a, b in zip((th, m, v, p), copies):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))
    # clean gradient: the whole step equals stats + apply with flag 0
    x16[1234] = 0
    st, flag, ssq = orc.shard_adam_step(x16, th, m, v, p, step=5, lr=LR, beta1=B1, beta2=B2,
                                        eps=EPS, inv_scale=S16)
    ref = _apply(orc, x16, copies[0], copies[1], copies[2], 5)
    assert st == 0 and flag == 0
    for a, b in zip((th, m, v, p), ref):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))
    assert ssq == orc.grad_stats(x16, S16)[1]


def test_apply_with_overflow_flag_writes_nothing(orc):
    rng = np.random.default_rng(14)
    n = 3000
    th = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m = (rng.standard_normal(n) * 1e-4).astype(np.float32)
    v = np.abs(rng.standard_normal(n) * 1e-6).astype(np.float32)
    x16 = _f16(rng.standard_normal(n) * 65.536)
    got = _apply(orc, x16, th, m, v, 4, overflow=1)
    for a, b in zip(got[:3], (th, m, v)):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))
    assert not got[3].any()


def test_loss_scale_invariance(orc):
    # only g = x * s enters the update: x * 2^k with s * 2^-k gives the same bits
    rng = np.random.default_rng(12)
    n = 4000
    th0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m0 = (rng.standard_normal(n) * 1e-4).astype(np.float32)
    v0 = np.abs(rng.standard_normal(n) * 1e-6).astype(np.float32)
    base = rng.standard_normal(n) * 1e-3
    a = _apply(orc, _f16(base * 2 ** 12), th0, m0, v0, 3, s=2.0 ** -12)
    b = _apply(orc, _f16(base * 2 ** 14), th0, m0, v0, 3, s=2.0 ** -14)
    for i in range(4):
        assert np.array_equal(a[i].view(np.uint8), b[i].view(np.uint8))


def test_fp32_gradient_matches_fp16_gradient(orc):
    # the fp32-gradient entry computes the same update when the fp32 gradient
    # holds the same values as the fp16 one
    rng = np.random.default_rng(13)
    n = 3000
    th0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    x16 = _f16(rng.standard_normal(n) * 65.536)
    x32 = x16.view(np.float16).astype(np.float32)
    z = np.zeros(n, np.float32)
    a = _apply(orc, x16, th0, z, z, 1)
    b = _apply(orc, x32, th0, z, z, 1)
    for i in range(4):
        assert np.array_equal(a[i].view(np.uint8), b[i].view(np.uint8))
