"""Arrays longer than the part that the statistics and the reduce leave in
the Infinity Cache for the update: the statistics walk the gradient from its
end and load its first 256 MiB with the allocating cache policy and the rest
non-temporal, and the reduce writes the last 256 MiB of its fp32 sum with
sc1 and the rest non-temporal.  Both halves of each kernel run here, against
the oracle, with a non-finite value planted on either side of the boundary
in turn."""
import numpy as np
import pytest

import zero_partitioned_mixed_flat_amd as zs
from zero_partitioned_mixed_flat_amd import testkit as tk
from gpu_util import assert_stats, host_f32, host_u16, oracle_reduce_full, oracle_stats_full, require_gpu, say

pytestmark = pytest.mark.gpu

TAIL_BYTES = 256 << 20


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


@pytest.mark.parametrize("dtype", ["f16", "f32"])
def test_statistics_on_both_sides_of_the_cached_head(dev, dtype):
    import torch
    elem = 2 if dtype == "f16" else 4
    n = TAIL_BYTES // elem + 2_891_139      # the cached head, then a few thousand non-temporal tiles; ragged end
    boundary = TAIL_BYTES // elem
    s = 2.0 ** -16
    say(f"statistics across the cached head: {dtype}, n={n}, boundary={boundary}")
    if dtype == "f16":
        g = tk.normal_f16_(torch.empty(n, dtype=torch.float16, device=dev), 1e-3 * 65536, 0x7A, tk.STREAM_GRAD)
        host = host_u16
    else:
        g = tk.normal_f32_(torch.empty(n, dtype=torch.float32, device=dev), 0.0, 1e-3 * 65536, 0x7A, tk.STREAM_GRAD)
        host = host_f32
    stats, ws = zs.new_stats(dev), zs.new_workspace(n, dev)
    zs.grad_stats(g, stats, inv_grad_scale=s, workspace=ws)
    assert_stats(zs.read_stats(stats), oracle_stats_full(host(g), s), f"{dtype} clean")
    for pos, value in ((boundary - 1, float("inf")), (boundary, float("nan")), (0, float("-inf")), (n - 1, float("nan"))):
        keep = g[pos].clone()
        g[pos] = value
        zs.grad_stats(g, stats, inv_grad_scale=s, workspace=ws)
        flag = zs.read_stats(stats)[0]
        g[pos] = keep
        assert flag == 1, f"{dtype}: non-finite value at {pos} not flagged"
    zs.grad_stats(g, stats, inv_grad_scale=s, workspace=ws)
    assert zs.read_stats(stats)[0] == 0


@pytest.mark.parametrize("with_stats", [True, False])
def test_reduce_on_both_sides_of_the_cached_tail(dev, with_stats):
    import torch
    n = TAIL_BYTES // 4 + 2_891_139
    N = 2
    s = 2.0 ** -18
    say(f"reduce across the cached tail: N={N}, n={n}, stats={with_stats}")
    slices = [tk.normal_f16_(torch.empty(n, dtype=torch.float16, device=dev), 1e-3 * 4096, 0x7B, tk.STREAM_GRAD + r)
              for r in range(N)]
    out = torch.empty(n, dtype=torch.float32, device=dev)
    stats = zs.new_stats(dev) if with_stats else None
    zs.grad_reduce(slices, out, stats=stats, inv_grad_scale=s)
    ref = oracle_reduce_full([host_u16(t) for t in slices])
    got = host_f32(out)
    bad = np.flatnonzero(got.view(np.uint32) != ref.view(np.uint32))
    assert bad.size == 0, f"{bad.size} sums differ, first at {bad[0]}"
    if with_stats:
        assert_stats(zs.read_stats(stats), oracle_stats_full(ref, s), "reduce across the cached tail")
        boundary = n - TAIL_BYTES // 4
        for pos in (boundary - 1, boundary):
            keep = slices[1][pos].clone()
            slices[1][pos] = float("inf")
            zs.grad_reduce(slices, out, stats=stats, inv_grad_scale=s)
            slices[1][pos] = keep
            assert zs.read_stats(stats)[0] == 1, f"infinity at {pos} not flagged"
            assert np.isinf(host_f32(out[pos:pos + 1])[0])
