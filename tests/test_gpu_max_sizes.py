"""Maximum sizes: arrays with more than 2^31 elements and a flat replica of
7.5e9 values (element offsets beyond 2^32), where any 32-bit index or offset
in a kernel or its launch would wrap.  Compared with the oracle on sampled
qwZ blocks (every element of each sampled block, so that the block scale is
checked as well as the codes) and, for the all-gather, on whole shards."""
import numpy as np
import pytest

import oracle
import zero_partitioned_mixed_flat_amd as zs
from zero_partitioned_mixed_flat_amd import testkit as tk
from gpu_util import (assert_state_parity, assert_stats, host_f32, host_u16, oracle_qwz_quantize_full,
                      oracle_stats_full, require_gpu, say)

pytestmark = pytest.mark.gpu

LR, BETAS, EPS = 1e-4, (0.9, 0.999), 1e-8
S16 = 2.0 ** -16
BIG = (1 << 31) + 4097          # 2,147,487,745 elements: more than 2^31, ragged last tile and qwZ block


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


@pytest.fixture(autouse=True)
def _free_cached_memory():
    import torch
    yield
    torch.cuda.empty_cache()


def _sample_blocks(n, count, seed):
    """Indices of every element of `count` stratified 256-value blocks, the
    first and the last blocks included (the last one is short)."""
    nb = -(-n // 256)
    rng = np.random.default_rng(seed)
    stride = nb // count
    blocks = np.arange(count, dtype=np.int64) * stride + rng.integers(0, stride, count)
    blocks = np.unique(np.concatenate([[0, 1, nb - 2, nb - 1], blocks]))
    idx = (blocks[:, None] * 256 + np.arange(256)[None, :]).reshape(-1)
    return blocks, idx[idx < n]


def _gather(idx_dev, *tensors):
    out = []
    for t in tensors:
        sel = t.index_select(0, idx_dev)
        out.append(host_u16(sel) if t.dtype.itemsize == 2 and t.is_floating_point() else
                   sel.cpu().numpy() if t.dtype.itemsize == 1 else host_f32(sel))
    return out


@pytest.mark.timeout(900)
def test_update_with_qwz_beyond_2_31_elements(dev):
    import torch
    n = BIG
    say(f"update + qwZ, n={n}: generating")
    master, m, v, p16 = tk.init_shard_state(n, 0xB16, zero_moments=False, device=dev)
    g = tk.normal_f16_(torch.empty(n, dtype=torch.float16, device=dev), 1e-3 * 65536, 0xB16, tk.STREAM_GRAD)
    codes = torch.empty(n, dtype=torch.int8, device=dev)
    scales = torch.empty(zs.qwz_scales_len(n), dtype=torch.float32, device=dev)
    blocks, idx = _sample_blocks(n, 20_000, 0xB16)
    idx_dev = torch.from_numpy(idx).to(dev)
    before = _gather(idx_dev, master, m, v, p16)
    stats, ws = zs.new_stats(dev), zs.new_workspace(n, dev)
    say("  GPU statistics + fused update")
    zs.grad_stats(g, stats, inv_grad_scale=S16, workspace=ws)
    zs.adam_step(g, master, m, v, p16, step=1000, lr=LR, betas=BETAS, eps=EPS, inv_grad_scale=S16,
                 stats=stats, stats_precomputed=True, qwz_codes=codes, qwz_scales=scales)
    got_stats = zs.read_stats(stats)
    say("  oracle statistics over the whole gradient")
    g_h = host_u16(g)
    ref_stats = oracle_stats_full(g_h, S16)
    assert_stats(got_stats, ref_stats, "2^31+ stats")
    assert ref_stats[0] == 0
    after = _gather(idx_dev, master, m, v, p16)
    ref = [a.copy() for a in before]
    assert oracle.adam_apply(g_h[idx], *ref, step=1000, lr=LR, beta1=BETAS[0], beta2=BETAS[1], eps=EPS,
                             inv_scale=S16, overflow=0) == 0
    assert sum(assert_state_parity(after, ref, "2^31+ sample").values()) == 0
    # the sampled blocks' codes and scales against the oracle's encoding of the
    # oracle's fp16 weights, block by block
    got_codes = codes.index_select(0, idx_dev).cpu().numpy()
    got_scales = scales.index_select(0, torch.from_numpy(blocks).to(dev)).cpu().numpy()
    pos = 0
    for b_i, b in enumerate(blocks):
        size = min(256, n - int(b) * 256)
        rc, rs = oracle.qwz_quantize(ref[3][pos:pos + size])
        assert np.array_equal(got_codes[pos:pos + size], rc), f"block {b}"
        assert got_scales[b_i].view(np.uint32) == rs[0].view(np.uint32), f"block {b}"
        pos += size
    assert pos == idx.size


@pytest.mark.timeout(900)
def test_encoder_beyond_2_31_values(dev):
    import torch
    n = BIG
    say(f"qwz_quantize, n={n}")
    x = tk.normal_f16_(torch.empty(n, dtype=torch.float16, device=dev), 0.02, 0xB17, tk.STREAM_MASTER)
    codes = torch.empty(n, dtype=torch.int8, device=dev)
    scales = torch.empty(zs.qwz_scales_len(n), dtype=torch.float32, device=dev)
    zs.qwz_quantize(x, codes, scales)
    blocks, idx = _sample_blocks(n, 50_000, 0xB17)
    idx_dev = torch.from_numpy(idx).to(dev)
    x_s = host_u16(x.index_select(0, idx_dev))
    got_codes = codes.index_select(0, idx_dev).cpu().numpy()
    got_scales = scales.index_select(0, torch.from_numpy(blocks).to(dev)).cpu().numpy()
    pos = 0
    for b_i, b in enumerate(blocks):
        size = min(256, n - int(b) * 256)
        rc, rs = oracle.qwz_quantize(x_s[pos:pos + size])
        assert np.array_equal(got_codes[pos:pos + size], rc), f"block {b}"
        assert got_scales[b_i].view(np.uint32) == rs[0].view(np.uint32), f"block {b}"
        pos += size


@pytest.mark.timeout(900)
def test_allgathers_of_a_7p5b_replica(dev):
    """psi = 7.5e9 from 64 shards of 117,187,584 (the last rank holds 5,376
    padding values): the fp16 all-gather compared in full, the qwZ all-gather
    compared on whole shards of ranks 0, 1, 37, 62 and 63."""
    import torch
    psi, N = 7_500_000_000, 64
    L = zs.partition_layout(psi, N, 0, 128).shard_len
    say(f"allgather psi={psi} N={N} shard_len={L}: generating")
    shards = [tk.normal_f16_(torch.empty(L, dtype=torch.float16, device=dev), 1.0, 0xB18, tk.STREAM_GRAD + r)
              for r in range(N)]
    replica = torch.empty(psi, dtype=torch.float16, device=dev)
    zs.allgather(shards, replica)
    say("  oracle all-gather")
    ref = oracle.allgather([host_u16(t) for t in shards], psi)
    assert np.array_equal(host_u16(replica), ref)
    del ref
    say("  qwZ: encode the shards, decode into the replica")
    codes, scales = [], []
    for t in shards:
        c = torch.empty(L, dtype=torch.int8, device=dev)
        s = torch.empty(zs.qwz_scales_len(L), dtype=torch.float32, device=dev)
        zs.qwz_quantize(t, c, s)
        codes.append(c)
        scales.append(s)
    replica.fill_(7.0)
    zs.qwz_allgather(codes, scales, replica)
    for r in (0, 1, 37, 62, 63):
        rc, rs = oracle_qwz_quantize_full(host_u16(shards[r]))
        real = min(L, psi - r * L)
        dec = oracle.qwz_dequantize(rc, rs)[:real]
        got = host_u16(replica[r * L:r * L + real])
        assert np.array_equal(got, dec), f"rank {r}"
        assert np.array_equal(codes[r].cpu().numpy(), rc), f"rank {r} codes"
