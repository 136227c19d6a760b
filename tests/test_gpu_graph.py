"""The path captured in a HIP graph (through torch.cuda.CUDAGraph) and
replayed: the library enqueues only kernels on the caller's stream (no
allocation, no memset, no host synchronisation), so a captured step must
give, replay after replay, the same bits as the same calls made eagerly,
and both must match the oracle.  Every replay is checked, with the eager
work and a synchronisation between replays."""
import numpy as np
import pytest

import oracle
import zero_partitioned_mixed_flat_amd as zs
from zero_partitioned_mixed_flat_amd import testkit as tk
from gpu_util import assert_state_parity, assert_stats, host_f32, host_u16, require_gpu, say

pytestmark = pytest.mark.gpu

LR, BETAS, EPS = 1e-4, (0.9, 0.999), 1e-8


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def _bits(t):
    import torch
    return t.view(torch.int16 if t.element_size() == 2 else torch.int32 if t.element_size() == 4 else torch.int8)


def _same(a, b):
    import torch
    return torch.equal(_bits(a), _bits(b))


def test_reduce_step_gather_replay(dev):
    """Reduce of 4 fp16 slices with fused statistics, the update with the
    qwZ encoder and global-norm clipping, and the decoding all-gather of
    this shard with three other encoded shards, captured once and replayed
    four times (the step number is part of the captured launch, so every
    replay applies t = 5)."""
    import torch
    N, L = 4, 262_144 + 512
    psi = N * L - 300
    say(f"graph: reduce N={N} + step + qwz gather, shard_len={L}")
    slices = [tk.normal_f16_(torch.empty(L, dtype=torch.float16, device=dev), 1e-3 * 65536, 0x6A, tk.STREAM_GRAD + r)
              for r in range(N)]
    init = tk.init_shard_state(L, 0x6A, zero_moments=False, device=dev)
    others, others_x = [], []
    for r in range(1, N):
        x = tk.normal_f16_(torch.empty(L, dtype=torch.float16, device=dev), 0.02, 0x6B, tk.STREAM_MASTER + r)
        c = torch.empty(L, dtype=torch.int8, device=dev)
        s = torch.empty(zs.qwz_scales_len(L), dtype=torch.float32, device=dev)
        zs.qwz_quantize(x, c, s)
        others.append((c, s))
        others_x.append(host_u16(x))

    def buffers():
        return dict(state=[t.clone() for t in init], gsum=torch.empty(L, dtype=torch.float32, device=dev),
                    stats=zs.new_stats(dev), ws=zs.new_workspace(L, dev),
                    codes=torch.empty(L, dtype=torch.int8, device=dev),
                    scales=torch.empty(zs.qwz_scales_len(L), dtype=torch.float32, device=dev),
                    replica=torch.empty(psi, dtype=torch.float16, device=dev))

    inv = 2.0 ** -16 / N

    def run(b):
        zs.grad_reduce(slices, b["gsum"], stats=b["stats"], inv_grad_scale=inv, workspace=b["ws"])
        zs.adam_step(b["gsum"], *b["state"], step=5, lr=LR, betas=BETAS, eps=EPS, inv_grad_scale=inv,
                     max_grad_norm=0.05, stats=b["stats"], stats_precomputed=True, qwz_codes=b["codes"],
                     qwz_scales=b["scales"])
        zs.qwz_allgather([b["codes"]] + [c for c, _ in others], [b["scales"]] + [s for _, s in others],
                         b["replica"])

    warm, cap, eager = buffers(), buffers(), buffers()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run(warm)                      # first calls fill the per-device caches outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run(cap)
    torch.cuda.synchronize()
    assert all(_same(a, b) for a, b in zip(cap["state"], init)), "capture must not execute the kernels"

    # the oracle's sequence: reduce, statistics, clipped update, encode, decode + gather
    ref = [host_f32(init[0]), host_f32(init[1]), host_f32(init[2]), host_u16(init[3])]
    ref_sum = oracle.grad_reduce([host_u16(t) for t in slices])
    # the other ranks' shards as the oracle encodes and decodes them
    other_dec = [oracle.qwz_dequantize(*oracle.qwz_quantize(x)) for x in others_x]
    for rep in range(4):
        graph.replay()
        run(eager)
        torch.cuda.synchronize()
        for name in ("gsum", "stats", "codes", "scales", "replica"):
            assert _same(cap[name], eager[name]), f"replay {rep}: {name} differs from the eager run"
        for a, b in zip(cap["state"], eager["state"]):
            assert _same(a, b), f"replay {rep}: state differs from the eager run"
        rc, rflag, rssq = oracle.shard_adam_step(ref_sum, *ref, step=5, lr=LR, beta1=BETAS[0], beta2=BETAS[1],
                                                 eps=EPS, inv_scale=inv, max_norm=0.05)
        assert rc == 0 and rflag == 0
        assert np.array_equal(host_f32(cap["gsum"]).view(np.uint32), ref_sum.view(np.uint32))
        assert_stats(zs.read_stats(cap["stats"]), (rflag, rssq), f"graph replay {rep}")
        got = [host_f32(cap["state"][0]), host_f32(cap["state"][1]), host_f32(cap["state"][2]),
               host_u16(cap["state"][3])]
        assert sum(assert_state_parity(got, ref, f"graph replay {rep}").values()) == 0
        rc_codes, rc_scales = oracle.qwz_quantize(ref[3])
        assert np.array_equal(cap["codes"].cpu().numpy(), rc_codes)
        assert np.array_equal(cap["scales"].cpu().numpy().view(np.uint32), rc_scales.view(np.uint32))
        want = oracle.allgather([oracle.qwz_dequantize(rc_codes, rc_scales)] + other_dec, psi)
        assert np.array_equal(host_u16(cap["replica"]), want)


def test_statistics_and_step_replay_match_eager_bench_shape(dev):
    """The benchmark's step (statistics, then the update gated on them)
    captured and replayed eight times on a 1,000,003-param shard."""
    import torch
    n = 1_000_003
    say(f"graph: stats + step, n={n}")
    init = tk.init_shard_state(n, 0x6C, zero_moments=False, device=dev)
    g = tk.normal_f16_(torch.empty(n, dtype=torch.float16, device=dev), 1e-3 * 65536, 0x6C, tk.STREAM_GRAD)
    cap = [t.clone() for t in init]
    eager = [t.clone() for t in init]
    st_c, ws_c = zs.new_stats(dev), zs.new_workspace(n, dev)
    st_e, ws_e = zs.new_stats(dev), zs.new_workspace(n, dev)

    def run(state, st, ws):
        zs.grad_stats(g, st, inv_grad_scale=2.0 ** -16, workspace=ws)
        zs.adam_step(g, *state, step=1000, lr=LR, betas=BETAS, eps=EPS, inv_grad_scale=2.0 ** -16, stats=st,
                     stats_precomputed=True)

    warm = [t.clone() for t in init]
    run(warm, zs.new_stats(dev), zs.new_workspace(n, dev))
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run(cap, st_c, ws_c)
    for rep in range(8):
        graph.replay()
        run(eager, st_e, ws_e)
        torch.cuda.synchronize()
        assert zs.read_stats(st_c) == zs.read_stats(st_e)
        for a, b in zip(cap, eager):
            assert _same(a, b), f"replay {rep}"
