"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (statistics call, then the update with the statistics
precomputed; or the reduce with fused statistics, then the update).  The
oracle runs on the CPU over the full arrays where that takes seconds, and on
stratified samples (plus the ragged tail) otherwise; the overflow flag always
comes from the oracle over the full gradient, except where noted.  Inputs
follow the workloads' recipes: master ~ N(0,0.02), m ~ N(0,1e-4),
v ~ |N(0,1e-6)|, fp16 gradients ~ N(0,1e-3) * loss scale (Student-t(3) *
1e-3 * 2^16 for the unpartitioned run); Adam lr 1e-4, betas (0.9, 0.999),
eps 1e-8."""
import numpy as np
import pytest

import oracle
import zero_partitioned_mixed_flat_amd as zs
from zero_partitioned_mixed_flat_amd import testkit as tk
from gpu_util import (assert_state_parity, assert_stats, host_f32, host_u16, oracle_apply_full,
                      oracle_qwz_dequantize_full, oracle_qwz_quantize_full, oracle_reduce_full,
                      oracle_stats_full, require_gpu, say, stratified_sample)

pytestmark = pytest.mark.gpu

LR, BETAS, EPS = 1e-4, (0.9, 0.999), 1e-8
S16 = 2.0 ** -16


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


@pytest.fixture(autouse=True)
def _free_cached_memory():
    import torch
    yield
    torch.cuda.empty_cache()


def _grad16(n, seed, dev, scale, stream=tk.STREAM_GRAD):
    import torch
    return tk.normal_f16_(torch.empty(n, dtype=torch.float16, device=dev), scale, seed, stream)


def _bench_step(g, master, m, v, p16, stats, ws, *, step, s):
    """The benchmark's step: statistics, then the update gated on them."""
    zs.grad_stats(g, stats, inv_grad_scale=s, workspace=ws)
    zs.adam_step(g, master, m, v, p16, step=step, lr=LR, betas=BETAS, eps=EPS, inv_grad_scale=s,
                 stats=stats, stats_precomputed=True)
    return zs.read_stats(stats)


def _gather(idx_dev, *tensors):
    out = []
    for t in tensors:
        sel = t.index_select(0, idx_dev)
        out.append(host_u16(sel) if t.element_size() == 2 else host_f32(sel))
    return out


def _apply_sample(g_sample, state, *, step, s, overflow):
    assert oracle.adam_apply(g_sample, *state, step=step, lr=LR, beta1=BETAS[0], beta2=BETAS[1], eps=EPS,
                             inv_scale=s, overflow=overflow) == 0


@pytest.mark.timeout(600)
def test_gpt2xl_shard_full_arrays(dev):
    """psi = 1.5e9, N = 4, rank 0 (375,000,064 params), t = 1000; every
    element compared."""
    import torch
    lay = zs.partition_layout(1_500_000_000, 4, 0, 128)
    n = lay.shard_len
    say(f"GPT-2-XL shard: n={n}, generating")
    master, m, v, p16 = tk.init_shard_state(n, 0xC2, zero_moments=False, device=dev)
    g = _grad16(n, 0xC2, dev, 1e-3 * 65536)
    torch.cuda.synchronize()
    g_h = host_u16(g)
    ref = [host_f32(master), host_f32(m), host_f32(v), host_u16(p16)]
    stats, ws = zs.new_stats(dev), zs.new_workspace(n, dev)
    say("  GPU step")
    got_stats = _bench_step(g, master, m, v, p16, stats, ws, step=1000, s=S16)
    say("  oracle statistics and update")
    ref_stats = oracle_stats_full(g_h, S16)
    assert_stats(got_stats, ref_stats, "gpt2xl")
    oracle_apply_full(g_h, *ref, step=1000, lr=LR, betas=BETAS, eps=EPS, s=S16, overflow=ref_stats[0])
    say("  compare")
    counts = assert_state_parity([host_f32(master), host_f32(m), host_f32(v), host_u16(p16)], ref, "gpt2xl")
    say("  inexact elements:", counts)
    assert sum(counts.values()) == 0


@pytest.mark.timeout(600)
def test_gpt2xl_shard_clipped_sampled(dev):
    """The GPT-2-XL shard with global-norm clipping at max_norm = 1 (the
    shard's gradient norm is about 19): compared on a stratified sample, with
    the device statistics set to the oracle's sum of squares so that the
    clipping factor is the same on both sides."""
    import struct

    import torch
    n = zs.partition_layout(1_500_000_000, 4, 0, 128).shard_len
    say(f"GPT-2-XL shard, clipped: n={n}")
    master, m, v, p16 = tk.init_shard_state(n, 0xC2C, zero_moments=False, device=dev)
    g = _grad16(n, 0xC2C, dev, 1e-3 * 65536)
    idx = stratified_sample(n, 2_000_000, 0xC2C)
    idx_dev = torch.from_numpy(idx).to(dev)
    before = _gather(idx_dev, master, m, v, p16)
    g_h = host_u16(g)
    flag, ssq = oracle_stats_full(g_h, S16)
    assert flag == 0 and np.sqrt(ssq) > 1.0
    st = torch.from_numpy(np.frombuffer(struct.pack("<IId", flag, 0, ssq), dtype=np.uint8).copy()).to(dev)
    zs.adam_step(g, master, m, v, p16, step=1000, lr=LR, betas=BETAS, eps=EPS, inv_grad_scale=S16,
                 max_grad_norm=1.0, stats=st, stats_precomputed=True)
    after = _gather(idx_dev, master, m, v, p16)
    ref = [a.copy() for a in before]
    _apply_sample(g_h[idx], ref, step=1000, s=S16 * oracle.clip_factor(ssq, 1.0), overflow=0)
    counts = assert_state_parity(after, ref, "gpt2xl clipped sample")
    assert sum(counts.values()) == 0


@pytest.mark.timeout(600)
def test_gpt2xl_allgather_full(dev):
    """The flat fp16 replica of psi = 1.5e9 from the four ranks' 375,000,064
    shards (the last ends with 256 padding values, not copied); every element
    compared."""
    import torch
    psi, N = 1_500_000_000, 4
    L = zs.partition_layout(psi, N, 0, 128).shard_len
    say(f"allgather psi={psi} N={N} shard_len={L}")
    shards = [_grad16(L, 0xA6, dev, 1.0, tk.STREAM_GRAD + r) for r in range(N)]
    replica = torch.empty(psi, dtype=torch.float16, device=dev)
    zs.allgather(shards, replica)
    ref = oracle.allgather([host_u16(t) for t in shards], psi)
    assert np.array_equal(host_u16(replica), ref)


@pytest.mark.timeout(600)
def test_gpt2xl_shard_qwz_full_arrays(dev):
    """The GPT-2-XL shard's update with the qwZ encoder fused into the
    write-back (the benchmark's launch: statistics, then the update with
    them precomputed); every state element, code and scale compared with
    the oracle's step followed by the oracle's encoding."""
    import torch
    n = zs.partition_layout(1_500_000_000, 4, 0, 128).shard_len
    say(f"GPT-2-XL shard, fused qwZ: n={n}, generating")
    master, m, v, p16 = tk.init_shard_state(n, 0xC2F, zero_moments=False, device=dev)
    g = _grad16(n, 0xC2F, dev, 1e-3 * 65536)
    torch.cuda.synchronize()
    g_h = host_u16(g)
    ref = [host_f32(master), host_f32(m), host_f32(v), host_u16(p16)]
    stats, ws = zs.new_stats(dev), zs.new_workspace(n, dev)
    codes = torch.empty(n, dtype=torch.int8, device=dev)
    scales = torch.empty(zs.qwz_scales_len(n), dtype=torch.float32, device=dev)
    say("  GPU step")
    zs.grad_stats(g, stats, inv_grad_scale=S16, workspace=ws)
    zs.adam_step(g, master, m, v, p16, step=1000, lr=LR, betas=BETAS, eps=EPS, inv_grad_scale=S16,
                 stats=stats, stats_precomputed=True, qwz_codes=codes, qwz_scales=scales)
    got_stats = zs.read_stats(stats)
    say("  oracle step and encoding")
    ref_stats = oracle_stats_full(g_h, S16)
    assert_stats(got_stats, ref_stats, "gpt2xl qwz")
    oracle_apply_full(g_h, *ref, step=1000, lr=LR, betas=BETAS, eps=EPS, s=S16, overflow=ref_stats[0])
    rc, rs = oracle_qwz_quantize_full(ref[3])
    say("  compare")
    counts = assert_state_parity([host_f32(master), host_f32(m), host_f32(v), host_u16(p16)], ref, "gpt2xl qwz")
    assert sum(counts.values()) == 0
    assert np.array_equal(scales.cpu().numpy().view(np.uint32), rs.view(np.uint32))
    assert np.array_equal(codes.cpu().numpy(), rc)


@pytest.mark.timeout(600)
def test_gpt2xl_qwz_allgather_full(dev):
    """The quantized all-gather of psi = 1.5e9 from the four ranks' encoded
    375,000,064 shards: every code, scale and replica element compared."""
    import torch
    psi, N = 1_500_000_000, 4
    L = zs.partition_layout(psi, N, 0, 128).shard_len
    say(f"qwz allgather psi={psi} N={N} shard_len={L}")
    codes, scales, ref_dec = [], [], []
    for r in range(N):
        x = tk.normal_f16_(torch.empty(L, dtype=torch.float16, device=dev), 0.02, 0xA7, tk.STREAM_MASTER + r)
        c = torch.empty(L, dtype=torch.int8, device=dev)
        s = torch.empty(zs.qwz_scales_len(L), dtype=torch.float32, device=dev)
        zs.qwz_quantize(x, c, s)
        rc, rs = oracle_qwz_quantize_full(host_u16(x))
        del x
        assert np.array_equal(s.cpu().numpy().view(np.uint32), rs.view(np.uint32))
        assert np.array_equal(c.cpu().numpy(), rc)
        ref_dec.append(oracle_qwz_dequantize_full(rc, rs))
        codes.append(c)
        scales.append(s)
    replica = torch.empty(psi, dtype=torch.float16, device=dev)
    zs.qwz_allgather(codes, scales, replica)
    ref = oracle.allgather(ref_dec, psi)
    assert np.array_equal(host_u16(replica), ref)


@pytest.mark.timeout(900)
def test_7b_n8_shard_full_and_inf_run(dev):
    """psi = 7e9, N = 8, rank 0 (875,000,064 params), t = 1000: a clean run
    compared element by element over the full arrays, then a run with
    0.001% of the gradient set to +inf whose step must be skipped with every
    state bit unchanged."""
    import torch
    lay = zs.partition_layout(7_000_000_000, 8, 0, 128)
    n = lay.shard_len
    say(f"7B/N=8 shard: n={n}, generating")
    master, m, v, p16 = tk.init_shard_state(n, 0xC4, zero_moments=False, device=dev)
    g = _grad16(n, 0xC4, dev, 1e-3 * 65536)
    torch.cuda.synchronize()
    g_h = host_u16(g)
    ref = [host_f32(master), host_f32(m), host_f32(v), host_u16(p16)]
    stats, ws = zs.new_stats(dev), zs.new_workspace(n, dev)
    say("  GPU step (clean)")
    got = _bench_step(g, master, m, v, p16, stats, ws, step=1000, s=S16)
    say("  oracle statistics and update over the full arrays")
    ref_stats = oracle_stats_full(g_h, S16)
    assert_stats(got, ref_stats, "7b clean")
    assert ref_stats[0] == 0
    oracle_apply_full(g_h, *ref, step=1000, lr=LR, betas=BETAS, eps=EPS, s=S16, overflow=0)
    say("  compare")
    counts = assert_state_parity([host_f32(master), host_f32(m), host_f32(v), host_u16(p16)], ref, "7b clean")
    say("  inexact elements:", counts)
    assert sum(counts.values()) == 0
    del ref

    say("  GPU step (+inf run)")
    tk.inject_inf_f16_(g, 1e-5, 0xC4F)
    g_h = host_u16(g)
    n_inf = int((g_h == 0x7C00).sum())
    say(f"  injected +inf entries: {n_inf}")
    assert n_inf > 0
    snapshot = [t.clone() for t in (master, m, v, p16)]
    flag, _ = _bench_step(g, master, m, v, p16, stats, ws, step=1001, s=S16)
    assert flag == oracle_stats_full(g_h, S16)[0] == 1
    for a, b in zip((master, m, v, p16), snapshot):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))


@pytest.mark.timeout(600)
def test_7p5b_n64_reduce_then_step(dev):
    """psi = 7.5e9, N = 64 (117,187,584 params): 64 simulated fp16 slices
    ~ N(0,1e-3)*2^12 summed on the owner, then the step at t = 10 on the
    fp32 sum with s = 2^-12/64; the sum, the statistics and every state
    element compared."""
    import torch
    lay = zs.partition_layout(7_500_000_000, 64, 0, 128)
    n = lay.shard_len
    say(f"7.5B/N=64 shard: n={n}, generating 64 slices")
    slices = [_grad16(n, 0xC3, dev, 1e-3 * 4096, tk.STREAM_GRAD + r) for r in range(64)]
    master, m, v, p16 = tk.init_shard_state(n, 0xC3, zero_moments=False, device=dev)
    s = 2.0 ** -12 / 64
    gsum = torch.empty(n, dtype=torch.float32, device=dev)
    stats, ws = zs.new_stats(dev), zs.new_workspace(n, dev)
    ref = [host_f32(master), host_f32(m), host_f32(v), host_u16(p16)]
    say("  GPU reduce + step")
    zs.grad_reduce(slices, gsum, stats=stats, inv_grad_scale=s, workspace=ws)
    red_stats = zs.read_stats(stats)
    zs.adam_step(gsum, master, m, v, p16, step=10, lr=LR, betas=BETAS, eps=EPS, inv_grad_scale=s,
                 stats=stats, stats_precomputed=True)
    say("  oracle reduce (full)")
    slices_h = [host_u16(t) for t in slices]
    del slices
    ref_sum = oracle_reduce_full(slices_h)
    del slices_h
    assert np.array_equal(host_f32(gsum).view(np.uint32), ref_sum.view(np.uint32))
    ref_stats = oracle_stats_full(ref_sum, s)
    assert_stats(red_stats, ref_stats, "7.5b reduce")
    say("  oracle update (full)")
    oracle_apply_full(ref_sum, *ref, step=10, lr=LR, betas=BETAS, eps=EPS, s=s, overflow=ref_stats[0])
    counts = assert_state_parity([host_f32(master), host_f32(m), host_f32(v), host_u16(p16)], ref, "7.5b step")
    say("  inexact elements:", counts)
    assert sum(counts.values()) == 0


@pytest.mark.timeout(900)
def test_unpartitioned_100_steps_drift(dev):
    """psi = 1.5e9 at N = 1 (the 16*psi case), the labelled drift run: 100
    Adam steps t = 1..100 from m = v = 0 with fresh seeded Student-t(3) *
    1e-3 * 2^16 gradients in which every draw whose fp16 would overflow is
    redrawn, so that every step applies; compared on a 1,048,576-param
    stratified sample.  The overflow flag and sum of squares are checked
    against the oracle over the full gradient at steps 1, 25, 50, 75, 100 (in
    between, the oracle's flag is the sample's, and any disagreement would
    show in the compared states).  The literal run, with the gradients as
    drawn, is the next test."""
    import torch
    n = 1_500_000_000
    lay = zs.partition_layout(n, 1, 0, 128)
    assert lay.shard_len == n and lay.real_len == n
    say(f"unpartitioned drift run: n={n}, generating state")
    master, m, v, p16 = tk.init_shard_state(n, 0xC5, zero_moments=True, device=dev)
    g = torch.empty(n, dtype=torch.float16, device=dev)
    stats, ws = zs.new_stats(dev), zs.new_workspace(n, dev)
    idx = stratified_sample(n, 1_048_576, 0xC5, edge=0)
    idx_dev = torch.from_numpy(idx).to(dev)
    ref = _gather(idx_dev, master, m, v, p16)
    t = 0
    for k in range(100):
        tk.student_t3_f16_(g, 1e-3 * 65536, 0xC5, tk.STREAM_GRAD + k, redraw_overflow=True)
        g_s = host_u16(g.index_select(0, idx_dev))
        flag, ssq = _bench_step(g, master, m, v, p16, stats, ws, step=t + 1, s=S16)
        if k % 25 == 24 or k == 0:
            rflag, rssq = oracle_stats_full(host_u16(g), S16)
            assert_stats((flag, ssq), (rflag, rssq), f"drift step {k + 1}")
            say(f"  step {k + 1}: full-gradient flag {rflag}, sumsq {rssq:.6e}")
        else:
            rflag = oracle.grad_stats(g_s, S16)[0]
        assert flag == rflag == 0
        _apply_sample(g_s, ref, step=t + 1, s=S16, overflow=rflag)
        t += 1
        if k in (0, 9, 49, 99):
            counts = assert_state_parity(_gather(idx_dev, master, m, v, p16), ref, f"drift step {k + 1}")
            say(f"  step {k + 1}: sample inexact {counts}")
            assert sum(counts.values()) == 0


@pytest.mark.timeout(1200)
def test_unpartitioned_100_literal_steps(dev):
    """psi = 1.5e9 at N = 1, the workload as written: 100 consecutive steps,
    each with a fresh seeded Student-t(3) * 1e-3 * 2^16 gradient taken as
    drawn (no redraw; about 3.3 entries per step overflow fp16, so most steps
    are skipped).  At every step the GPU's overflow flag must equal the
    oracle's over the full 1.5e9-value gradient (and the sum of squares, on
    steps that apply); t advances only on applied steps; the states are
    compared with the oracle's on a 1,048,576-param stratified sample after
    steps 10, 50 and 100 (a skipped step must leave them unchanged, which the
    oracle's gated update does)."""
    import torch
    n = 1_500_000_000
    say(f"unpartitioned literal run: n={n}, generating state")
    master, m, v, p16 = tk.init_shard_state(n, 0xC5, zero_moments=True, device=dev)
    g = torch.empty(n, dtype=torch.float16, device=dev)
    # the full gradient comes to the host every step: one pinned buffer
    g_pinned = torch.empty(n, dtype=torch.int16, pin_memory=True)
    g_host = g_pinned.numpy().view(np.uint16)
    stats, ws = zs.new_stats(dev), zs.new_workspace(n, dev)
    idx = stratified_sample(n, 1_048_576, 0xC51, edge=0)
    idx_dev = torch.from_numpy(idx).to(dev)
    ref = _gather(idx_dev, master, m, v, p16)
    t = 0
    applied = []
    for k in range(100):
        tk.student_t3_f16_(g, 1e-3 * 65536, 0xC5, tk.STREAM_GRAD + 2000 + k, redraw_overflow=False)
        g_pinned.copy_(g.view(torch.int16))
        flag, ssq = _bench_step(g, master, m, v, p16, stats, ws, step=t + 1, s=S16)
        rflag, rssq = oracle_stats_full(g_host, S16)
        assert_stats((flag, ssq), (rflag, rssq), f"literal step {k + 1}")
        _apply_sample(g_host[idx], ref, step=t + 1, s=S16, overflow=rflag)
        if rflag == 0:
            t += 1
            applied.append(k + 1)
        n_inf = int(torch.count_nonzero((g.view(torch.int16) & 0x7FFF) == 0x7C00))  # for the log only
        say(f"  literal step {k + 1}: flag {flag}, fp16 infinities {n_inf}, applied so far {len(applied)}")
        if k + 1 in (10, 50, 100):
            counts = assert_state_parity(_gather(idx_dev, master, m, v, p16), ref, f"literal step {k + 1}")
            say(f"  after step {k + 1}: sample inexact {counts}")
            assert sum(counts.values()) == 0
    say(f"  literal run: {len(applied)} of 100 steps applied (steps {applied})")
