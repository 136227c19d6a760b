"""GPU parity of the HIP library (through its C ABI) against the CPU oracle on
the same seeded inputs, at sizes the oracle finishes in seconds: ragged
lengths across several tiles, the tiny workload end to end, the reduce for
N = 1..64, and the invariants (skip on overflow, determinism, separability,
padding).  The bar: flag bit-exact, fp32 rel <= 1e-6, fp16 <= 1 ulp,
sum of squares rel <= 1e-10; the expected design result is bit-exact and
each test also reports the count of inexact elements."""
import numpy as np
import pytest

import oracle
import zero_partitioned_mixed_flat_amd as zs
from zero_partitioned_mixed_flat_amd import probes, testkit as tk
from gpu_util import (assert_state_parity, assert_stats, host_f32, host_u16, require_gpu, say)

pytestmark = pytest.mark.gpu

LR, BETAS, EPS = 1e-4, (0.9, 0.999), 1e-8
S16 = 2.0 ** -16


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def _state(n, seed, zero_moments, dev):
    return tk.init_shard_state(n, seed, zero_moments=zero_moments, device=dev)


def _grad16(n, seed, dev, scale=1e-3 * 65536, stream=tk.STREAM_GRAD):
    import torch
    return tk.normal_f16_(torch.empty(n, dtype=torch.float16, device=dev), scale, seed, stream)


def _host_state(master, m, v, p16):
    return [host_f32(master), host_f32(m), host_f32(v), host_u16(p16)]


def _oracle_step(g_host, st, *, step, s):
    master, m, v, p16 = [a.copy() for a in st]
    rc, flag, ssq = oracle.shard_adam_step(g_host, master, m, v, p16, step=step, lr=LR, beta1=BETAS[0],
                                           beta2=BETAS[1], eps=EPS, inv_scale=s)
    assert rc == 0
    return (master, m, v, p16), (flag, ssq)


def _gpu_step(g, master, m, v, p16, *, step, s, stats=None, precomputed=False):
    stats = zs.new_stats(g.device) if stats is None else stats
    zs.adam_step(g, master, m, v, p16, step=step, lr=LR, betas=BETAS, eps=EPS, inv_grad_scale=s,
                 stats=stats, stats_precomputed=precomputed)
    return zs.read_stats(stats)


LENGTHS = [1, 3, 4, 5, 7, 255, 256, 1023, 1024, 4095, 4096, 4097, 8191, 65536 + 13, 262_144,
           1_000_003]


@pytest.mark.parametrize("n", LENGTHS)
@pytest.mark.parametrize("step,zero_moments", [(1, True), (1000, False)])
def test_step_f16_grad(dev, n, step, zero_moments):
    seed = 1000 + n
    say(f"adam_step f16 n={n} step={step} seed={seed}")
    master, m, v, p16 = _state(n, seed, zero_moments, dev)
    g = _grad16(n, seed, dev)
    before = _host_state(master, m, v, p16)
    g_h = host_u16(g)
    ref_state, ref_stats = _oracle_step(g_h, before, step=step, s=S16)
    got_stats = _gpu_step(g, master, m, v, p16, step=step, s=S16)
    assert_stats(got_stats, ref_stats, f"n={n}")
    counts = assert_state_parity(_host_state(master, m, v, p16), ref_state, f"n={n}")
    say("  inexact elements:", counts)
    assert sum(counts.values()) == 0, "expected bit-exact parity"


@pytest.mark.parametrize("n", [1, 6, 4097, 100_003])
def test_step_f32_grad(dev, n):
    import torch
    seed = 2000 + n
    say(f"adam_step f32 n={n} seed={seed}")
    master, m, v, p16 = _state(n, seed, False, dev)
    g = tk.normal_f32_(torch.empty(n, dtype=torch.float32, device=dev), 0.0, 4 * 1e-3 * 65536, seed,
                       tk.STREAM_GRAD)
    before = _host_state(master, m, v, p16)
    ref_state, ref_stats = _oracle_step(host_f32(g), before, step=10, s=2.0 ** -18)
    got_stats = _gpu_step(g, master, m, v, p16, step=10, s=2.0 ** -18)
    assert_stats(got_stats, ref_stats, f"f32 n={n}")
    counts = assert_state_parity(_host_state(master, m, v, p16), ref_state, f"f32 n={n}")
    assert sum(counts.values()) == 0


def test_tiny_workload_end_to_end(dev):
    """Psi = 1,048,576, N = 4, rank 0 owns 262,144 (align 128); four simulated
    ranks' fp16 gradients ~ N(0,1e-3)*2^16 are summed on the owner, then one
    Adam step at t = 1 from m = v = 0 with s = 2^-16/4 (the mean enters
    through the scale)."""
    import torch
    lay = zs.partition_layout(1_048_576, 4, 0, 128)
    assert tuple(lay) == oracle.partition_layout(1_048_576, 4, 0, 128)[1]
    n = lay.shard_len
    assert n == 262_144
    seed = 0xC1
    say(f"tiny workload: reduce N=4 + step, n={n}")
    slices = [_grad16(n, seed, dev, stream=tk.STREAM_GRAD + r) for r in range(4)]
    master, m, v, p16 = _state(n, seed, True, dev)
    s = 2.0 ** -16 / 4
    gsum = torch.empty(n, dtype=torch.float32, device=dev)
    stats = zs.new_stats(dev)
    zs.grad_reduce(slices, gsum, stats=stats, inv_grad_scale=s)
    red_stats = zs.read_stats(stats)
    before = _host_state(master, m, v, p16)
    slices_h = [host_u16(t) for t in slices]
    ref_sum = oracle.grad_reduce(slices_h)
    assert np.array_equal(host_f32(gsum).view(np.uint32), ref_sum.view(np.uint32))
    assert_stats(red_stats, oracle.grad_stats(ref_sum, s), "tiny reduce")
    _gpu_step(gsum, master, m, v, p16, step=1, s=s, stats=stats, precomputed=True)
    ref_state, _ = _oracle_step(ref_sum, before, step=1, s=s)
    counts = assert_state_parity(_host_state(master, m, v, p16), ref_state, "tiny")
    say("  inexact:", counts)
    assert sum(counts.values()) == 0
    # t = 1 from m = v = 0: the step is the closed form theta - lr*g/(|g|+eps)
    g = ref_sum.astype(np.float64) * s
    closed = before[0].astype(np.float64) - LR * g / (np.abs(g) + EPS)
    th = host_f32(master).astype(np.float64)
    assert (np.abs(th - closed) <= np.spacing(np.abs(host_f32(master))) / 2 + 8 * 2.0 ** -24 * LR).all()


def _stats_tensor(dev, flag, sumsq):
    """A device zero_grad_stats_t holding given values (e.g. statistics
    summed over ranks, as an all-reduce would deliver them)."""
    import struct

    import torch
    raw = np.frombuffer(struct.pack("<IId", flag, 0, sumsq), dtype=np.uint8).copy()
    return torch.from_numpy(raw).to(dev)


@pytest.mark.parametrize("n,max_norm", [(4097, 0.01), (300_001, 0.1), (300_001, 1e9)])
def test_clipping_with_given_global_stats(dev, n, max_norm):
    """Clipping reads the device statistics; given the oracle's own (or the
    sum over four shards, standing in for the all-reduce), the GPU step is
    bit-identical to the oracle's."""
    seed = 3000 + n
    say(f"adam_step clip n={n} max_norm={max_norm}")
    master, m, v, p16 = _state(n, seed, False, dev)
    g = _grad16(n, seed, dev)
    before = _host_state(master, m, v, p16)
    g_h = host_u16(g)
    flag, ssq = oracle.grad_stats(g_h, S16)
    other = [oracle.grad_stats(host_u16(_grad16(n, seed, dev, stream=tk.STREAM_GRAD + 1 + r)), S16)[1]
             for r in range(3)]
    for total in (ssq, ssq + sum(other)):
        st = _stats_tensor(dev, flag, total)
        gm, gv, gt, gp = [t.clone() for t in (m, v, master, p16)]
        zs.adam_step(g, gt, gm, gv, gp, step=7, lr=LR, betas=BETAS, eps=EPS, inv_grad_scale=S16,
                     max_grad_norm=max_norm, stats=st, stats_precomputed=True)
        ref = [a.copy() for a in before]
        scale = S16 * oracle.clip_factor(total, max_norm)
        assert oracle.adam_apply(g_h, *ref, step=7, lr=LR, beta1=BETAS[0], beta2=BETAS[1], eps=EPS,
                                 inv_scale=scale, overflow=flag) == 0
        counts = assert_state_parity(_host_state(gt, gm, gv, gp), ref, f"clip n={n}")
        assert sum(counts.values()) == 0


def test_clipping_end_to_end(dev):
    """Statistics computed by the GPU, clipping active.  The GPU's and the
    oracle's sums of squares may differ in the last bits (summation order);
    the clipped step depends on them only through the binary32 multiplier
    (float)(inv_scale * max_norm / sqrt(sumsq)).  For this input both sums
    give the same multiplier (asserted), so the step is bit-exact."""
    n = 250_003
    master, m, v, p16 = _state(n, 31, False, dev)
    g = _grad16(n, 31, dev)
    before = _host_state(master, m, v, p16)
    g_h = host_u16(g)
    stats = zs.new_stats(dev)
    zs.adam_step(g, master, m, v, p16, step=2, lr=LR, betas=BETAS, eps=EPS, inv_grad_scale=S16,
                 max_grad_norm=0.05, stats=stats)
    got_stats = zs.read_stats(stats)
    ref = [a.copy() for a in before]
    rc, rflag, rssq = oracle.shard_adam_step(g_h, *ref, step=2, lr=LR, beta1=BETAS[0], beta2=BETAS[1], eps=EPS,
                                             inv_scale=S16, max_norm=0.05)
    assert rc == 0 and np.sqrt(rssq) > 0.05
    assert_stats(got_stats, (rflag, rssq), "clip e2e")
    mult = [np.float32(S16 * oracle.clip_factor(x, 0.05)) for x in (got_stats[1], rssq)]
    assert mult[0] == mult[1], f"clip multipliers differ: {mult}"
    counts = assert_state_parity(_host_state(master, m, v, p16), ref, "clip e2e")
    say("  inexact elements:", counts)
    assert sum(counts.values()) == 0


@pytest.mark.parametrize("n_slices", [1, 2, 3, 8, 9, 17, 64])
@pytest.mark.parametrize("n", [5, 2048, 2049, 70_001])
def test_reduce(dev, n_slices, n):
    import torch
    seed = 31 * n_slices + n
    say(f"grad_reduce N={n_slices} n={n} seed={seed}")
    slices = [_grad16(n, seed, dev, scale=1e-3 * 4096, stream=tk.STREAM_GRAD + r) for r in range(n_slices)]
    out = torch.empty(n, dtype=torch.float32, device=dev)
    stats = zs.new_stats(dev)
    s = 2.0 ** -12 / n_slices
    zs.grad_reduce(slices, out, stats=stats, inv_grad_scale=s)
    ref = oracle.grad_reduce([host_u16(t) for t in slices])
    assert np.array_equal(host_f32(out).view(np.uint32), ref.view(np.uint32))
    assert_stats(zs.read_stats(stats), oracle.grad_stats(ref, s), f"reduce N={n_slices}")
    out2 = torch.empty(n, dtype=torch.float32, device=dev)
    zs.grad_reduce(slices, out2)            # without statistics
    assert torch.equal(out, out2)


def test_reduce_many_partials(dev):
    """More than 4096 tiles: the partials are folded in two levels."""
    import torch
    n, N = 4096 * 1024 + 777, 3
    say(f"grad_reduce N={N} n={n} (two-level fold)")
    slices = [_grad16(n, 99, dev, stream=tk.STREAM_GRAD + r) for r in range(N)]
    out = torch.empty(n, dtype=torch.float32, device=dev)
    stats = zs.new_stats(dev)
    zs.grad_reduce(slices, out, stats=stats, inv_grad_scale=2.0 ** -18)
    ref = oracle.grad_reduce([host_u16(t) for t in slices])
    assert np.array_equal(host_f32(out).view(np.uint32), ref.view(np.uint32))
    assert_stats(zs.read_stats(stats), oracle.grad_stats(ref, 2.0 ** -18), "reduce two-level fold")
    slices[2][n - 1] = float("inf")
    zs.grad_reduce(slices, out, stats=stats, inv_grad_scale=2.0 ** -18)
    assert zs.read_stats(stats)[0] == 1


@pytest.mark.parametrize("psi,n_ranks", [(1, 1), (1000, 4), (1_000_003, 4), (1_048_576, 4), (777_777, 64),
                                          (5000, 64), (4095, 3)])
def test_allgather(dev, psi, n_ranks):
    """The flat fp16 replica from N shards: ragged last shards, empty shards
    (psi small against N), N = 64."""
    import torch
    lay = zs.partition_layout(psi, n_ranks, 0, 128)
    L = lay.shard_len
    say(f"allgather psi={psi} N={n_ranks} shard_len={L}")
    shards = [_grad16(L, psi, dev, stream=tk.STREAM_GRAD + r) for r in range(n_ranks)]
    replica = torch.empty(psi, dtype=torch.float16, device=dev)
    zs.allgather(shards, replica)
    ref = oracle.allgather([host_u16(t) for t in shards], psi)
    assert np.array_equal(host_u16(replica), ref)


@pytest.mark.parametrize("special", [np.inf, -np.inf, np.nan])
def test_reduce_flags_nonfinite_slice(dev, special):
    import torch
    n, N = 9000, 5
    slices = [_grad16(n, 77, dev, stream=tk.STREAM_GRAD + r) for r in range(N)]
    slices[3][4321] = float(special)
    out = torch.empty(n, dtype=torch.float32, device=dev)
    stats = zs.new_stats(dev)
    zs.grad_reduce(slices, out, stats=stats, inv_grad_scale=2.0 ** -18)
    ref = oracle.grad_reduce([host_u16(t) for t in slices])
    got = host_f32(out)
    keep = np.ones(n, dtype=bool)
    keep[4321] = False
    assert np.array_equal(got.view(np.uint32)[keep], ref.view(np.uint32)[keep])
    assert np.isnan(got[4321]) == np.isnan(ref[4321]) and (np.isnan(ref[4321]) or got[4321] == ref[4321])
    assert zs.read_stats(stats)[0] == 1 == oracle.grad_stats(ref, 2.0 ** -18)[0]


@pytest.mark.parametrize("special,pos", [(np.inf, 0), (-np.inf, 131_071), (np.nan, 77_777)])
def test_overflow_skips_step(dev, special, pos):
    n = 131_072
    master, m, v, p16 = _state(n, 5, False, dev)
    g = _grad16(n, 5, dev)
    g[pos] = float(special)
    before = _host_state(master, m, v, p16)
    flag, _ = _gpu_step(g, master, m, v, p16, step=3, s=S16)
    ref_state, (ref_flag, _) = _oracle_step(host_u16(g), before, step=3, s=S16)
    assert flag == ref_flag == 1
    after = _host_state(master, m, v, p16)
    for a, b in zip(after, before):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))


def test_inf_injection_run(dev):
    n = 500_000
    g = _grad16(n, 0xC4, dev)
    tk.inject_inf_f16_(g, 1e-5, 0xC4F)
    g_h = host_u16(g)
    n_inf = int((g_h == 0x7C00).sum())
    say(f"injected +inf count: {n_inf}")
    master, m, v, p16 = _state(n, 0xC4, False, dev)
    before = _host_state(master, m, v, p16)
    flag, _ = _gpu_step(g, master, m, v, p16, step=1000, s=S16)
    assert flag == oracle.grad_stats(g_h, S16)[0] == (1 if n_inf else 0)
    if n_inf:
        for a, b in zip(_host_state(master, m, v, p16), before):
            assert np.array_equal(a.view(np.uint8), b.view(np.uint8))


def test_deterministic(dev):
    import torch
    n = 300_001
    outs = []
    for _ in range(2):
        master, m, v, p16 = _state(n, 42, False, dev)
        g = _grad16(n, 42, dev)
        st = _gpu_step(g, master, m, v, p16, step=17, s=S16)
        outs.append((st, [t.clone() for t in (master, m, v, p16)]))
    assert outs[0][0] == outs[1][0]            # flag and sumsq bit-identical
    for a, b in zip(outs[0][1], outs[1][1]):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))


def test_sharded_equals_unsharded(dev):
    """Fact 1 of "DeepSpeed ZeRO Stages" 2.1: updating shards separately is
    exactly the update of the whole; the shard views come from the layout."""
    import torch
    psi, N = 1_000_000, 4
    lay = [zs.partition_layout(psi, N, r, 128) for r in range(N)]
    total = lay[0].psi_padded
    master, m, v, p16 = _state(total, 9, False, dev)
    g = _grad16(total, 9, dev)
    whole = [t.clone() for t in (master, m, v, p16)]
    _gpu_step(g, *whole, step=5, s=S16)
    for L in lay:
        sl = slice(L.offset, L.offset + L.shard_len)
        _gpu_step(g[sl], master[sl], m[sl], v[sl], p16[sl], step=5, s=S16)
    for a, b in zip((master, m, v, p16), whole):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))


def test_padding_stays_zero(dev):
    import torch
    lay = zs.partition_layout(1_500_001, 4, 3, 128)
    n, real = lay.shard_len, lay.real_len
    assert n > real
    master, m, v, p16 = _state(n, 3, False, dev)
    g = _grad16(n, 3, dev)
    for t in (master, m, v, p16, g):
        t[real:] = 0
    _gpu_step(g, master, m, v, p16, step=2, s=S16)
    for t in (master, m, v, p16):
        assert not t[real:].view(torch.uint8).any()


def test_zero_length(dev):
    import torch
    e32 = torch.empty(0, dtype=torch.float32, device=dev)
    e16 = torch.empty(0, dtype=torch.float16, device=dev)
    stats = zs.new_stats(dev)
    stats.fill_(0xFF)
    zs.adam_step(e16, e32, e32.clone(), e32.clone(), e16.clone(), step=1, lr=LR, stats=stats)
    assert zs.read_stats(stats) == (0, 0.0)
    stats.fill_(0xFF)
    zs.grad_reduce([e16, e16.clone()], e32.clone(), stats=stats)
    assert zs.read_stats(stats) == (0, 0.0)


def test_misaligned_view_is_rejected(dev):
    import torch
    master, m, v, p16 = _state(64, 1, False, dev)
    g = _grad16(64, 1, dev)
    with pytest.raises(zs.ZeroError) as e:
        _gpu_step(g[1:], master[1:], m[1:], v[1:], p16[1:], step=1, s=S16)
    assert e.value.status == -2
    with pytest.raises(zs.ZeroError):
        _gpu_step(g, master, m, v, p16, step=0, s=S16)
    out = torch.empty(63, dtype=torch.float32, device=dev)
    with pytest.raises(zs.ZeroError):
        zs.grad_reduce([g[1:]], out)


def test_generator_matches_host_philox(dev):
    n = 4096
    got = tk.philox(n, 0x1234_5678_9ABC_DEF0, 7).cpu().numpy().view(np.uint32).reshape(n, 4)
    ctr = np.zeros((n, 4), dtype=np.uint32)
    ctr[:, 0] = np.arange(n, dtype=np.uint32)
    ctr[:, 2] = 7
    ref = tk.philox_host(ctr, (0x9ABC_DEF0, 0x1234_5678))
    assert np.array_equal(got, ref)


def test_generator_moments(dev):
    import torch
    n = 1 << 22
    x = tk.normal_f32_(torch.empty(n, dtype=torch.float32, device=dev), 0.0, 1.0, 11, 1).double().cpu().numpy()
    se = 1 / np.sqrt(n)
    assert abs(x.mean()) < 5 * se and abs(x.std() - 1) < 5 * se
    from scipy.stats import t as student_t
    t3 = tk.student_t3_f16_(torch.empty(n, dtype=torch.float16, device=dev), scale=1.0, seed=12, stream=2)
    t3 = t3.float().cpu().numpy().astype(np.float64)
    # tail mass beyond 2 of Student-t with 3 degrees of freedom, from scipy
    want = 2 * student_t.sf(2.0, 3)
    p = (np.abs(t3) > 2).mean()
    assert abs(p - want) < 5 * np.sqrt(want * (1 - want) / n)


def test_device_arithmetic_matches_host_ieee(dev):
    """The library's primitives under its build flags: binary32 division and
    square root correctly rounded, binary32 -> binary16 round to nearest
    even with subnormals and overflow to inf, binary16 -> binary32 exact; on
    2^24 random bit patterns (every class: subnormals, infinities, NaNs) plus
    edge values, against numpy's IEEE results on the host."""
    import torch
    rng = np.random.default_rng(0xA417)
    n = 1 << 24
    a = rng.integers(0, 2**32, n, dtype=np.uint64).astype(np.uint32).view(np.float32)
    b = rng.integers(0, 2**32, n, dtype=np.uint64).astype(np.uint32).view(np.float32)
    edge = np.array([0.0, -0.0, 1.0, -1.0, 2.0 ** -149, 2.0 ** -126, 2.0 ** -126 - 2.0 ** -149, 3.4028235e38,
                     np.inf, -np.inf, np.nan, 65504.0, 65519.996, 65520.0, 2.0 ** -24, 2.0 ** -25,
                     2.0 ** -25 * (1 + 2.0 ** -23), 1.5 * 2.0 ** -24, 2.5 * 2.0 ** -24, 6.1035156e-05,
                     6.097555e-05, 0.1, 1e-8, 0.999], dtype=np.float32)
    m = edge.size
    a[:m * m] = np.repeat(edge, m)
    b[:m * m] = np.tile(edge, m)
    # small exact-value ranges where ties and subnormals are dense
    a[m * m:m * m + 65536] = np.arange(65536, dtype=np.float32) * np.float32(2.0 ** -25)
    h = rng.integers(0, 2**16, n, dtype=np.uint32).astype(np.uint16)
    h[:65536] = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    dev_a, dev_b = torch.from_numpy(a).to(dev), torch.from_numpy(b).to(dev)
    dev_h = torch.from_numpy(h.view(np.int16)).to(dev)
    quot, root, half, wide = probes.arith_f32(dev_a, dev_b, dev_h)
    with np.errstate(all="ignore"):
        want = {"quot": a / b, "root": np.sqrt(a), "half": a.astype(np.float16), "wide": h.view(np.float16).astype(np.float32)}
    got = {"quot": quot.cpu().numpy(), "root": root.cpu().numpy(),
           "half": half.cpu().numpy().view(np.float16), "wide": wide.cpu().numpy()}
    for name in want:
        w, g = want[name], got[name]
        nan_w, nan_g = np.isnan(w), np.isnan(g)
        assert np.array_equal(nan_w, nan_g), f"{name}: NaN positions differ"
        ui = np.uint16 if w.dtype == np.float16 else np.uint32
        bad = np.flatnonzero((w.view(ui) != g.view(ui)) & ~nan_w)
        assert bad.size == 0, f"{name}: {bad.size} mismatches; first at {bad[0]}: {g[bad[0]]!r} vs {w[bad[0]]!r}"


@pytest.mark.parametrize("step", [1, 7, 1000])
def test_zero_gradient_with_zero_moments_is_a_no_op(dev, step):
    """g = 0 and m = v = 0: every update term is 0, so the master weights keep
    their bits, the moments stay +0 and the fp16 copy is f16(master)."""
    import torch
    n = 100_003
    master, m, v, p16 = _state(n, 77, True, dev)
    before = _host_state(master, m, v, p16)
    g = torch.zeros(n, dtype=torch.float16, device=dev)
    flag, ssq = _gpu_step(g, master, m, v, p16, step=step, s=S16)
    assert (flag, ssq) == (0, 0.0)
    after = _host_state(master, m, v, p16)
    assert np.array_equal(after[0].view(np.uint32), before[0].view(np.uint32))
    assert not after[1].view(np.uint32).any() and not after[2].view(np.uint32).any()
    ref_state, _ = _oracle_step(host_u16(g), before, step=step, s=S16)
    assert np.array_equal(after[3], ref_state[3])
    assert np.array_equal(after[3], before[0].astype(np.float16).view(np.uint16))


def test_concurrent_calls_from_two_threads_on_two_streams(dev):
    """The library keeps no per-call state: two host threads, each with its
    own stream and buffers, run statistics + update steps at the same time
    and each ends with the oracle's result."""
    import threading

    import torch
    n = 300_001
    jobs = []
    for i in range(2):
        master, m, v, p16 = _state(n, 90 + i, False, dev)
        g = _grad16(n, 90 + i, dev)
        jobs.append(dict(state=[master, m, v, p16], g=g, before=_host_state(master, m, v, p16),
                         g_h=host_u16(g), stream=torch.cuda.Stream(), stats=zs.new_stats(dev),
                         ws=zs.new_workspace(n, dev), err=None))
    torch.cuda.synchronize()

    def work(job):
        try:
            with torch.cuda.stream(job["stream"]):
                for t in range(1, 6):
                    zs.grad_stats(job["g"], job["stats"], inv_grad_scale=S16, workspace=job["ws"])
                    zs.adam_step(job["g"], *job["state"], step=t, lr=LR, betas=BETAS, eps=EPS, inv_grad_scale=S16,
                                 stats=job["stats"], stats_precomputed=True)
            job["stream"].synchronize()
        except Exception as e:  # reported below, on the test's thread
            job["err"] = e

    threads = [threading.Thread(target=work, args=(job,)) for job in jobs]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    for i, job in enumerate(jobs):
        assert job["err"] is None, job["err"]
        ref = [a.copy() for a in job["before"]]
        for t in range(1, 6):
            rc, flag, _ = oracle.shard_adam_step(job["g_h"], *ref, step=t, lr=LR, beta1=BETAS[0], beta2=BETAS[1],
                                                 eps=EPS, inv_scale=S16)
            assert rc == 0 and flag == 0
        counts = assert_state_parity(_host_state(*job["state"]), ref, f"thread {i}")
        assert sum(counts.values()) == 0


def test_ceiling_kernels_compute_what_they_claim(dev):
    """The reference kernels behind the benchmark's ceiling: the copy copies,
    the in-place read-modify-write adds 1 to every element of whole 16-byte
    chunks and leaves a ragged tail alone, and the read sums its input."""
    import torch
    n = 1_000_003
    src = tk.normal_f32_(torch.empty(n, dtype=torch.float32, device=dev), 0.0, 1.0, 0x77, tk.STREAM_MASTER)
    dst = torch.empty_like(src)
    tk.copy_f32(src, dst)
    assert torch.equal(src, dst)
    before = host_f32(dst)
    probes.rmw_f32(dst)
    after = host_f32(dst)
    body = (n // 4) * 4
    assert np.array_equal(after[:body], (before[:body] + np.float32(1.0)).astype(np.float32))
    assert np.array_equal(after[body:], before[body:])
    sink = torch.zeros(1 << 16, dtype=torch.float32, device=dev)
    tk.read_f32(src, sink)
    total = float(sink.double().sum())
    assert abs(total - float(src[:body].double().sum())) <= 1e-3 * float(src[:body].abs().double().sum())
    # the many-slice reference: every slice read (XOR over the per-block
    # results), and with an output the per-element XOR, ragged tail included
    ns = 1024 * 37 + 12
    sl = [_grad16(ns, 0x78, dev, stream=tk.STREAM_GRAD + r) for r in range(7)]
    want = np.zeros(ns, dtype=np.uint32)
    for t in sl:
        want ^= host_u16(t).astype(np.uint32)
    xsink = torch.zeros(64, dtype=torch.int32, device=dev)
    tk.read_slices(sl, xsink)
    got = np.bitwise_xor.reduce(xsink.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(want)
    out = torch.full((ns,), -1, dtype=torch.int32, device=dev)
    xsink.zero_()
    tk.read_slices(sl, xsink, out)
    assert np.array_equal(out.cpu().numpy().view(np.uint32), want)
    assert np.bitwise_xor.reduce(xsink.cpu().numpy().view(np.uint32)) == np.bitwise_xor.reduce(want)


def test_explicit_stream_without_workspace(dev):
    """Calls given another stream and no workspace allocate a temporary one
    that the caching allocator must not hand out again before that stream
    has used it: tensors allocated and filled right after the calls on the
    current stream must not disturb the statistics, and the results must
    equal those of the same calls on the current stream."""
    import torch
    n = 300_001
    g = _grad16(n, 0x57, dev)
    slices = [_grad16(n, 0x57, dev, stream=tk.STREAM_GRAD + 1 + r) for r in range(4)]
    a = list(_state(n, 0x57, False, dev))
    b = [t.clone() for t in a]
    sa, sb, sr, srb = (zs.new_stats(dev) for _ in range(4))
    out_a = torch.empty(n, dtype=torch.float32, device=dev)
    out_b = torch.empty_like(out_a)
    kw = dict(step=5, lr=LR, betas=BETAS, eps=EPS, inv_grad_scale=S16, max_grad_norm=0.05)
    zs.adam_step(g, *a, stats=sa, **kw)
    zs.grad_reduce(slices, out_a, stats=sr, inv_grad_scale=S16 / 4)
    ga = zs.new_stats(dev)
    zs.grad_stats(g, ga, inv_grad_scale=S16)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    gb = zs.new_stats(dev)
    zs.adam_step(g, *b, stats=sb, stream=side, **kw)
    zs.grad_reduce(slices, out_b, stats=srb, inv_grad_scale=S16 / 4, stream=side)
    zs.grad_stats(g, gb, inv_grad_scale=S16, stream=side)
    # allocations on the current stream right away: without the recorded
    # stream they could reuse the temporaries while the side stream runs
    junk = [torch.full((zs.workspace_bytes(n),), 0x7F, dtype=torch.uint8, device=dev) for _ in range(8)]
    side.synchronize()
    torch.cuda.synchronize()
    del junk
    for x, y in ((sa, sb), (sr, srb), (ga, gb)):
        assert zs.read_stats(x) == zs.read_stats(y)
    assert torch.equal(out_a.view(torch.int32), out_b.view(torch.int32))
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.uint8), y.view(torch.uint8))
