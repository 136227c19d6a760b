"""The multi-core SIMD host step (include/zero_host_adam.h; the CPU Adam of
ZeRO-Offload, "DeepSpeed ZeRO Stages" 5.1) against the oracle on the CPU:
the same bar as the GPU library's (bit-exact states and flag, sum of squares
within 1e-10 relative), for every instruction set level this CPU has, for
several thread counts, f16 and f32 gradients, ragged lengths, the skip on
overflow, clipping, and fp16 subnormal gradients.  Inputs are seeded numpy
draws with the workloads' distributions."""
import numpy as np
import pytest

from zero_partitioned_mixed_flat_amd import host_adam as ha
from gpu_util import assert_state_parity, assert_stats

LR, BETAS, EPS = 1e-4, (0.9, 0.999), 1e-8
S16 = 2.0 ** -16
BEST = ha.set_isa(0)
ISAS = list(range(ha.ISA_SCALAR, BEST + 1))


@pytest.fixture(autouse=True)
def _restore_isa():
    yield
    ha.set_isa(0)


def _state(n, seed, zero_moments=False):
    rng = np.random.default_rng(seed)
    master = (rng.standard_normal(n) * 0.02).astype(np.float32)
    if zero_moments:
        m = np.zeros(n, np.float32)
        v = np.zeros(n, np.float32)
    else:
        m = (rng.standard_normal(n) * 1e-4).astype(np.float32)
        v = np.abs(rng.standard_normal(n) * 1e-6).astype(np.float32)
    return [master, m, v, np.zeros(n, np.uint16)]


def _grad16(n, seed, scale=1e-3 * 65536):
    return (np.random.default_rng(seed + 1).standard_normal(n) * scale).astype(np.float16).view(np.uint16)


def _oracle(orc, g, st, *, step, s, max_norm=0.0):
    ref = [a.copy() for a in st]
    rc, flag, ssq = orc.shard_adam_step(g, *ref, step=step, lr=LR, beta1=BETAS[0], beta2=BETAS[1], eps=EPS,
                                        inv_scale=s, max_norm=max_norm)
    assert rc == 0
    return ref, (flag, ssq)


def _host(g, st, *, step, s, threads=0, max_norm=0.0, stats=None):
    out = [a.copy() for a in st]
    got = ha.adam_step(g, *out, step=step, lr=LR, betas=BETAS, eps=EPS, inv_grad_scale=s,
                       max_grad_norm=max_norm, stats=stats, threads=threads)
    return out, got


@pytest.mark.parametrize("isa", ISAS)
@pytest.mark.parametrize("n", [1, 15, 16, 17, 1000, 65536, 65537, 300_001])
def test_matches_oracle_f16(orc, isa, n):
    assert ha.set_isa(isa) == isa
    st = _state(n, n)
    g = _grad16(n, n)
    ref, ref_stats = _oracle(orc, g, st, step=1000, s=S16)
    got, got_stats = _host(g, st, step=1000, s=S16)
    assert_stats(got_stats, ref_stats, f"host isa={isa} n={n}")
    assert sum(assert_state_parity(got, ref, f"host isa={isa} n={n}").values()) == 0


@pytest.mark.parametrize("isa", ISAS)
def test_matches_oracle_f32_zero_moments(orc, isa):
    ha.set_isa(isa)
    n = 100_003
    st = _state(n, 5, zero_moments=True)
    g = (np.random.default_rng(6).standard_normal(n) * 1e-3).astype(np.float32)
    ref, ref_stats = _oracle(orc, g, st, step=1, s=1.0)
    got, got_stats = _host(g, st, step=1, s=1.0)
    assert_stats(got_stats, ref_stats, "host f32")
    assert sum(assert_state_parity(got, ref, "host f32").values()) == 0


def test_subnormal_gradients(orc):
    """fp16 subnormal gradients are converted exactly, and the tiny unscaled
    values go through the update without flushing."""
    n = 40_000
    st = _state(n, 7, zero_moments=True)
    k = np.random.default_rng(8).integers(-1023, 1024, n)
    g = (k * 2.0 ** -24).astype(np.float16).view(np.uint16)
    ref, ref_stats = _oracle(orc, g, st, step=1, s=2.0 ** -10)
    for isa in ISAS:
        ha.set_isa(isa)
        got, got_stats = _host(g, st, step=1, s=2.0 ** -10)
        assert_stats(got_stats, ref_stats, f"subnormal isa={isa}")
        assert sum(assert_state_parity(got, ref, f"subnormal isa={isa}").values()) == 0


def test_same_bits_for_every_isa_and_thread_count():
    n = 3 * 65536 + 1234
    st = _state(n, 9)
    g = _grad16(n, 9)
    base = None
    for isa in ISAS:
        ha.set_isa(isa)
        for threads in (1, 2, 3, 8):
            got, stats = _host(g, st, step=50, s=S16, threads=threads)
            key = [a.tobytes() for a in got] + [np.float64(stats[1]).tobytes()]
            if base is None:
                base = key
            assert key == base, f"isa={isa} threads={threads}"


def _p16_at(n, byte_offset):
    """A uint16 array of n zeros starting byte_offset bytes past a 64-byte
    boundary (odd offsets give an unaligned array)."""
    raw = np.zeros(2 * n + 128, np.uint8)
    start = (-raw.ctypes.data) % 64 + byte_offset
    out = np.frombuffer(raw[start:start + 2 * n].data, dtype=np.uint16)
    assert out.ctypes.data % 64 == byte_offset
    return out


@pytest.mark.parametrize("byte_offset", [0, 2, 14, 30, 62])
@pytest.mark.parametrize("n", [5, 40, 65536 + 77])
def test_fp16_copy_at_any_alignment(orc, byte_offset, n):
    """The SIMD loops stream the fp16 copy with stores that need 16- or
    32-byte alignment: the elements before the first aligned address go
    through the scalar path."""
    st = _state(n, 11)
    g = _grad16(n, 11)
    ref, _ = _oracle(orc, g, st, step=77, s=S16)
    for isa in ISAS:
        ha.set_isa(isa)
        out = [a.copy() for a in st[:3]] + [_p16_at(n, byte_offset)]
        ha.adam_step(g, *out, step=77, lr=LR, betas=BETAS, eps=EPS, inv_grad_scale=S16, threads=3)
        assert sum(assert_state_parity(out, ref, f"isa={isa} offset={byte_offset} n={n}").values()) == 0


@pytest.mark.parametrize("special,pos", [(np.inf, 0), (-np.inf, 65_535), (np.nan, 123_457)])
def test_overflow_skips(orc, special, pos):
    n = 200_000
    st = _state(n, 11)
    g = _grad16(n, 11)
    g[pos] = np.array([special], dtype=np.float16).view(np.uint16)[0]
    for isa in ISAS:
        ha.set_isa(isa)
        got, (flag, _) = _host(g, st, step=3, s=S16)
        assert flag == 1
        for a, b in zip(got, st):
            assert np.array_equal(a.view(np.uint8), b.view(np.uint8))
    assert orc.grad_stats(g, S16)[0] == 1


def test_clipping(orc):
    n = 250_003
    st = _state(n, 12)
    g = _grad16(n, 12)
    flag, ssq = orc.grad_stats(g, S16)
    assert flag == 0 and np.sqrt(ssq) > 0.05
    ref, _ = _oracle(orc, g, st, step=2, s=S16, max_norm=0.05)
    # with the oracle's statistics handed in, the clipping factor is the same
    got, _ = _host(g, st, step=2, s=S16, max_norm=0.05, stats=(flag, ssq))
    assert sum(assert_state_parity(got, ref, "host clip, given stats").values()) == 0
    # with its own statistics: within the parity bar
    got2, stats2 = _host(g, st, step=2, s=S16, max_norm=0.05)
    assert_stats(stats2, (flag, ssq), "host clip")
    assert_state_parity(got2, ref, "host clip")


def test_misaligned_arrays_rejected():
    n = 64
    st = _state(n, 12)
    g = _grad16(n, 12)
    with pytest.raises(ha.HostAdamError, match="aligned"):
        ha.adam_step(g, *st[:3], _p16_at(n, 1), step=1, lr=LR)
    raw = np.zeros(4 * n + 8, np.uint8)
    master_odd = np.frombuffer(raw[2:2 + 4 * n].data, dtype=np.float32)
    if master_odd.ctypes.data % 4:
        with pytest.raises(ha.HostAdamError, match="aligned"):
            ha.adam_step(g, master_odd, *st[1:], step=1, lr=LR)


def test_zero_length_and_errors():
    e32, e16 = np.zeros(0, np.float32), np.zeros(0, np.uint16)
    assert ha.adam_step(e16, e32, e32.copy(), e32.copy(), e16.copy(), step=1, lr=LR) == (0, 0.0)
    st = _state(10, 1)
    g = _grad16(10, 1)
    for kw in (dict(step=0), dict(lr=-1.0), dict(betas=(1.0, 0.9)), dict(eps=0.0), dict(inv_grad_scale=0.0),
               dict(max_grad_norm=-1.0), dict(threads=-1)):
        args = dict(step=1, lr=LR)
        args.update(kw)
        with pytest.raises(ha.HostAdamError):
            ha.adam_step(g, *[a.copy() for a in st], **args)
    with pytest.raises(ha.HostAdamError):
        ha.adam_step(g, st[0], st[0], st[2], st[3], step=1, lr=LR)      # master aliases exp_avg
    with pytest.raises(ha.HostAdamError):
        ha.set_isa(4)
