"""The step with its step number held in device memory
(zero_shard_adam_step_device_t): the device-side bias corrections against
the oracle's, a sequence of steps with a skipped (overflowing) one, which
must not advance t, and the step captured once in a HIP graph and replayed
step after step with fresh gradients, each replay checked against the
oracle's sequence."""
import numpy as np
import pytest

import oracle
import zero_partitioned_mixed_flat_amd as zs
from zero_partitioned_mixed_flat_amd import probes, testkit as tk
from gpu_util import assert_state_parity, assert_stats, host_f32, host_u16, require_gpu, say

pytestmark = pytest.mark.gpu

LR, BETAS, EPS = 1e-4, (0.9, 0.999), 1e-8
S16 = 2.0 ** -16


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


@pytest.mark.parametrize("beta", [0.9, 0.999, 0.95, 0.99, 0.9999, 0.5])
def test_device_bias_corrections_match_oracle(dev, beta):
    """(float)(1 - beta^t) formed on the device equals the oracle's host
    value for every t = 1..65536 and for 65,536 seeded t up to 10^9."""
    import torch
    rng = np.random.default_rng(int(beta * 1e4))
    t = np.concatenate([np.arange(1, 65537), rng.integers(65537, 10**9, 65536)]).astype(np.int64)
    got = probes.bias_correction(beta, torch.from_numpy(t).to(dev)).cpu().numpy()
    want = np.empty(t.size, dtype=np.float32)
    for i, tt in enumerate(t):
        st, s = oracle.adam_scalars(LR, beta, 0.5, EPS, 1.0, int(tt))
        assert st == 0
        want[i] = s[4]
    bad = np.flatnonzero(got.view(np.uint32) != want.view(np.uint32))
    assert bad.size == 0, f"{bad.size} mismatches, first t={t[bad[0]]}: {got[bad[0]]!r} vs {want[bad[0]]!r}"


def _fresh_grad(g, seed):
    tk.normal_f16_(g, 1e-3 * 65536, seed, tk.STREAM_GRAD)


def _assert_counter(counter, applied, t_call, where):
    """The counter after a call numbered t_call: its count, and the two bias
    corrections it holds, which must be the oracle's for t_call."""
    raw = counter.cpu().numpy()
    assert int(raw[0]) == applied, f"{where}: counted {int(raw[0])}, want {applied}"
    bc = raw[1:2].view(np.float32)
    st, s = oracle.adam_scalars(LR, BETAS[0], BETAS[1], EPS, 1.0, t_call)
    assert st == 0
    assert bc.view(np.uint32).tolist() == s[4:6].view(np.uint32).tolist(), f"{where}: bias corrections {bc}"


@pytest.mark.parametrize("qwz", [False, True])
@pytest.mark.parametrize("max_norm", [0.0, 0.05])
def test_sequence_with_a_skipped_step(dev, qwz, max_norm):
    """Six steps with fresh gradients; the third overflows, so it writes
    nothing and t goes 1, 2, (skip), 3, 4, 5; the counter ends at 5.  With
    max_norm = 0.05 every applied step is clipped (the gradient's norm is
    about 0.3)."""
    import torch
    n = 100_003
    say(f"device t: sequence, n={n}, qwz={qwz}, max_norm={max_norm}")
    master, m, v, p16 = tk.init_shard_state(n, 0xD7, zero_moments=True, device=dev)
    ref = [host_f32(master), host_f32(m), host_f32(v), host_u16(p16)]
    g = torch.empty(n, dtype=torch.float16, device=dev)
    stats, ws, applied = zs.new_stats(dev), zs.new_workspace(n, dev), zs.new_step_counter(dev)
    codes = torch.empty(n, dtype=torch.int8, device=dev) if qwz else None
    scales = torch.empty(zs.qwz_scales_len(n), dtype=torch.float32, device=dev) if qwz else None
    t_ref = 0
    for k in range(6):
        _fresh_grad(g, 0xD70 + k)
        if k == 2:
            g[12345] = float("inf")
        g_h = host_u16(g)
        zs.adam_step_device_t(g, master, m, v, p16, applied_steps=applied, lr=LR, betas=BETAS, eps=EPS,
                              inv_grad_scale=S16, max_grad_norm=max_norm, stats=stats, workspace=ws,
                              qwz_codes=codes, qwz_scales=scales)
        got_stats = zs.read_stats(stats)
        flag, ssq = oracle.grad_stats(g_h, S16)
        if max_norm and not flag:
            assert oracle.clip_factor(ssq, max_norm) < 1.0, "the test means every applied step to be clipped"
        t_call = t_ref + 1
        if not flag:
            t_ref += 1
        rc, rflag, rssq = oracle.shard_adam_step(g_h, *ref, step=max(t_ref, 1), lr=LR, beta1=BETAS[0],
                                                 beta2=BETAS[1], eps=EPS, inv_scale=S16, max_norm=max_norm)
        assert rc == 0 and rflag == flag == (1 if k == 2 else 0)
        assert_stats(got_stats, (rflag, rssq), f"step {k}")
        _assert_counter(applied, t_ref, t_call, f"step {k}")
        counts = assert_state_parity([host_f32(master), host_f32(m), host_f32(v), host_u16(p16)], ref, f"step {k}")
        assert sum(counts.values()) == 0
        if qwz and not flag:
            rc_codes, rc_scales = oracle.qwz_quantize(ref[3])
            assert np.array_equal(codes.cpu().numpy(), rc_codes)
            assert np.array_equal(scales.cpu().numpy().view(np.uint32), rc_scales.view(np.uint32))
    assert t_ref == 5


@pytest.mark.parametrize("qwz", [False, True])
def test_fp32_gradient_sequence(dev, qwz):
    """fp32 gradients (the reduce's output) through the device-counter step:
    four steps, the second with a NaN, against the oracle's sequence."""
    import torch
    n = 70_001
    say(f"device t: fp32 gradient sequence, n={n}, qwz={qwz}")
    master, m, v, p16 = tk.init_shard_state(n, 0xD9, zero_moments=True, device=dev)
    ref = [host_f32(master), host_f32(m), host_f32(v), host_u16(p16)]
    g = torch.empty(n, dtype=torch.float32, device=dev)
    stats, ws, applied = zs.new_stats(dev), zs.new_workspace(n, dev), zs.new_step_counter(dev)
    codes = torch.empty(n, dtype=torch.int8, device=dev) if qwz else None
    scales = torch.empty(zs.qwz_scales_len(n), dtype=torch.float32, device=dev) if qwz else None
    s = 2.0 ** -18
    t_ref = 0
    for k in range(4):
        tk.normal_f32_(g, 0.0, 1e-3 / s, 0xD90 + k, tk.STREAM_GRAD)
        if k == 1:
            g[n // 2] = float("nan")
        g_h = host_f32(g)
        zs.adam_step_device_t(g, master, m, v, p16, applied_steps=applied, lr=LR, betas=BETAS, eps=EPS,
                              inv_grad_scale=s, stats=stats, workspace=ws, qwz_codes=codes, qwz_scales=scales)
        flag = oracle.grad_stats(g_h, s)[0]
        t_call = t_ref + 1
        t_ref += 0 if flag else 1
        rc, rflag, rssq = oracle.shard_adam_step(g_h, *ref, step=t_call, lr=LR, beta1=BETAS[0], beta2=BETAS[1],
                                                 eps=EPS, inv_scale=s)
        assert rc == 0 and rflag == flag == (1 if k == 1 else 0)
        assert_stats(zs.read_stats(stats), (rflag, rssq), f"fp32 step {k}")
        _assert_counter(applied, t_ref, t_call, f"fp32 step {k}")
        counts = assert_state_parity([host_f32(master), host_f32(m), host_f32(v), host_u16(p16)], ref,
                                     f"fp32 step {k}")
        assert sum(counts.values()) == 0
        if qwz and not flag:
            rc_codes, rc_scales = oracle.qwz_quantize(ref[3])
            assert np.array_equal(codes.cpu().numpy(), rc_codes)
            assert np.array_equal(scales.cpu().numpy().view(np.uint32), rc_scales.view(np.uint32))
    assert t_ref == 3


def test_empty_shard_still_counts_the_step(dev):
    """A rank whose shard is empty (psi small against N) still takes part in
    every step: with len = 0 the call writes no array but counts the step
    and stores that step's bias corrections, like every other rank."""
    import torch
    empty_f32 = torch.empty(0, dtype=torch.float32, device=dev)
    empty_f16 = torch.empty(0, dtype=torch.float16, device=dev)
    stats, ws, applied = zs.new_stats(dev), zs.new_workspace(0, dev), zs.new_step_counter(dev)
    for k in range(3):
        zs.adam_step_device_t(empty_f16, empty_f32, empty_f32.clone(), empty_f32.clone(), empty_f16.clone(),
                              applied_steps=applied, lr=LR, betas=BETAS, eps=EPS, inv_grad_scale=S16,
                              stats=stats, workspace=ws)
        assert zs.read_stats(stats) == (0, 0.0)
        _assert_counter(applied, k + 1, k + 1, f"empty shard, call {k}")


def test_graph_replayed_across_steps(dev):
    """Statistics + the device-t update captured once; before each replay
    the gradient buffer is refilled in place (eagerly) with the next step's
    gradient, one of them overflowing.  Eight replays, each against the
    oracle's step with its own t, then the counter."""
    import torch
    n = 262_144 + 77
    say(f"device t: graph replays, n={n}")
    master, m, v, p16 = tk.init_shard_state(n, 0xD8, zero_moments=False, device=dev)
    ref = [host_f32(master), host_f32(m), host_f32(v), host_u16(p16)]
    g = torch.empty(n, dtype=torch.float16, device=dev)
    stats, ws, applied = zs.new_stats(dev), zs.new_workspace(n, dev), zs.new_step_counter(dev)
    # first (eager) calls fill the library's per-device caches outside the capture
    warm = [t.clone() for t in (master, m, v, p16)]
    _fresh_grad(g, 1)
    zs.grad_stats(g, zs.new_stats(dev), inv_grad_scale=S16, workspace=zs.new_workspace(n, dev))
    zs.adam_step_device_t(g, *warm, applied_steps=zs.new_step_counter(dev), lr=LR, betas=BETAS, eps=EPS,
                          inv_grad_scale=S16, stats=zs.new_stats(dev), workspace=zs.new_workspace(n, dev))
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        zs.grad_stats(g, stats, inv_grad_scale=S16, workspace=ws)
        zs.adam_step_device_t(g, master, m, v, p16, applied_steps=applied, lr=LR, betas=BETAS, eps=EPS,
                              inv_grad_scale=S16, stats=stats, stats_precomputed=True)
    torch.cuda.synchronize()
    assert zs.read_step_counter(applied) == 0
    t_ref = 0
    for k in range(8):
        _fresh_grad(g, 0xD80 + k)
        if k == 4:
            g[n - 1] = float("-inf")
        g_h = host_u16(g)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        flag, ssq = oracle.grad_stats(g_h, S16)
        t_call = t_ref + 1
        t_ref += 0 if flag else 1
        assert_stats(zs.read_stats(stats), (flag, ssq), f"replay {k}")
        if not flag:
            assert oracle.adam_apply(g_h, *ref, step=t_ref, lr=LR, beta1=BETAS[0], beta2=BETAS[1], eps=EPS,
                                     inv_scale=S16, overflow=0) == 0
        _assert_counter(applied, t_ref, t_call, f"replay {k}")
        counts = assert_state_parity([host_f32(master), host_f32(m), host_f32(v), host_u16(p16)], ref,
                                     f"replay {k}")
        assert sum(counts.values()) == 0
    assert t_ref == 7
