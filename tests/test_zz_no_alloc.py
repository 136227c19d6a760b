"""zero_shard_adam_step_noalloc -- the step whose statistics use the
library's static per-device scratch instead of a caller's workspace --
against zero_shard_adam_step, called through the C ABI on the same inputs:
the statistics and every state bit must be identical.  The calls run in a
row on one device, each smaller than the one before, so that partials left
in the scratch by an earlier, larger call would show if a later call read
them: a clipped step (its factor depends on the sum of squares), a smaller
clipped step, a smaller step whose gradient holds one +inf (skipped), and a
smaller clean step after it (the flag must not stick)."""
import numpy as np
import pytest

import oracle
import zero_partitioned_mixed_flat_amd as zs
from zero_partitioned_mixed_flat_amd import testkit as tk
from gpu_util import assert_state_parity, assert_stats, host_f32, host_u16, require_gpu, say

pytestmark = pytest.mark.gpu

LR, BETAS, EPS, S16 = 1e-4, (0.9, 0.999), 1e-8, 2.0 ** -16


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def _state(n, seed, dev):
    master, m, v, p16 = tk.init_shard_state(n, seed, zero_moments=False, device=dev)
    return [master, m, v, p16]


def _host(ts):
    return [host_f32(ts[0]), host_f32(ts[1]), host_f32(ts[2]), host_u16(ts[3])]


# (length, seed, index of a planted +inf or None, max_grad_norm, step)
SEQUENCE = [
    (3_000_017, 0x5A1, None, 0.5, 11),
    (100_003, 0x5A2, None, 0.05, 12),
    (50_001, 0x5A3, 20_000, 0.0, 13),
    (4_099, 0x5A4, None, 0.0, 13),
]


def test_noalloc_matches_workspace_step_in_a_row(dev):
    import torch
    for n, seed, inf_at, max_norm, step in SEQUENCE:
        say(f"noalloc vs workspace step: n={n} seed={seed:#x} inf_at={inf_at} max_norm={max_norm} t={step}")
        g = tk.normal_f16_(torch.empty(n, dtype=torch.float16, device=dev), 1e-3 * 65536, seed, tk.STREAM_GRAD)
        if inf_at is not None:
            g[inf_at] = float("inf")
        a = _state(n, seed, dev)
        b = [t.clone() for t in a]
        before = _host(a)
        sa, sb = zs.new_stats(dev), zs.new_stats(dev)
        ws = zs.new_workspace(n, dev)
        kw = dict(step=step, lr=LR, betas=BETAS, eps=EPS, inv_grad_scale=S16, max_grad_norm=max_norm)
        zs.adam_step(g, *a, stats=sa, workspace=ws, **kw)
        zs.adam_step_noalloc(g, *b, stats=sb, **kw)
        got_a, got_b = zs.read_stats(sa), zs.read_stats(sb)
        # same kernels, same grid, same summation order: identical bits
        assert got_a[0] == got_b[0] == (1 if inf_at is not None else 0)
        if got_a[0] == 0:
            assert got_a[1] == got_b[1], f"sum of squares {got_a[1]!r} vs {got_b[1]!r}"
        ha, hb = _host(a), _host(b)
        for x, y, name in zip(ha, hb, ("master", "m", "v", "p16")):
            assert np.array_equal(x.view(np.uint8), y.view(np.uint8)), f"n={n}: {name} differs"
        # and both within the parity bar of the oracle's step
        ref = [x.copy() for x in before]
        rc, rflag, rssq = oracle.shard_adam_step(host_u16(g), *ref, step=step, lr=LR, beta1=BETAS[0],
                                                 beta2=BETAS[1], eps=EPS, inv_scale=S16, max_norm=max_norm)
        assert rc == 0
        assert_stats(got_b, (rflag, rssq), f"noalloc n={n}")
        counts = assert_state_parity(hb, ref, f"noalloc n={n}")
        say("  inexact elements against the oracle:", counts)
        if inf_at is not None:
            for x, y in zip(hb, before):
                assert np.array_equal(x.view(np.uint8), y.view(np.uint8))


def test_noalloc_with_precomputed_stats(dev):
    """With the statistics precomputed no scratch is used: the update alone,
    identical to the workspace entry point's."""
    import torch
    n = 70_001
    g = tk.normal_f16_(torch.empty(n, dtype=torch.float16, device=dev), 1e-3 * 65536, 0x5A5, tk.STREAM_GRAD)
    a = _state(n, 0x5A5, dev)
    b = [t.clone() for t in a]
    st = zs.new_stats(dev)
    zs.grad_stats(g, st, inv_grad_scale=S16)
    kw = dict(step=3, lr=LR, betas=BETAS, eps=EPS, inv_grad_scale=S16, stats=st, stats_precomputed=True)
    zs.adam_step(g, *a, **kw)
    zs.adam_step_noalloc(g, *b, **kw)
    for x, y in zip(_host(a), _host(b)):
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8))
