"""Both all-gathers on a shard with more tiles than one launch may have
blocks.  HIP takes a launch's size in work-items as a 32-bit count, so a grid
of 64-lane blocks stops at 67,108,863 blocks: with 512-value tiles, at
34,359,737,856 values of one shard.  The kernels walk the tiles beyond that
with a grid-stride loop.  One rank's shard of 34,359,740,416 values (68.7 GB
in fp16) with psi 100 values short of it (the last tile ragged); the replica
is compared with the oracle's all-gather (or the oracle's qwZ decoding) on
the first tiles, on every tile from the launch limit to the end, and on a
stratified sample, and the fp16 replica also element by element on the
device against its input."""
import numpy as np
import pytest

import oracle
from gpu_util import host_u16, require_gpu, say, stratified_sample

import zero_partitioned_mixed_flat_amd as zs
from zero_partitioned_mixed_flat_amd import testkit as tk

pytestmark = pytest.mark.gpu

LIMIT_VALUES = (0xFFFFFFFF // 64) * 512     # values covered by the largest launch
SHARD = LIMIT_VALUES + 5 * 512              # five tiles beyond it
PSI = SHARD - 100


# the fp16 case holds the shard and its replica at once (137 GB)
NEEDED_BYTES = 2 * 2 * SHARD + (8 << 30)


@pytest.fixture(scope="module")
def dev():
    import torch
    d = require_gpu()
    total = torch.cuda.get_device_properties(d).total_memory
    if total < NEEDED_BYTES:
        pytest.skip(f"needs {NEEDED_BYTES / 1e9:.0f} GB of device memory, the device has {total / 1e9:.0f} GB")
    return d


def _regions():
    head = (0, 1 << 20)
    tail = (LIMIT_VALUES - (1 << 20), PSI)
    return head, tail


@pytest.mark.timeout(900)
def test_fp16_allgather_beyond_launch_limit(dev):
    import torch
    torch.cuda.empty_cache()
    say(f"fp16 all-gather: shard {SHARD:,} values, psi {PSI:,}, launch limit at {LIMIT_VALUES:,}")
    shard = tk.normal_f16_(torch.empty(SHARD, dtype=torch.float16, device=dev), 1.0, 0xB1, tk.STREAM_GRAD)
    replica = torch.empty(PSI, dtype=torch.float16, device=dev)
    zs.allgather([shard], replica)
    torch.cuda.synchronize()
    for a, b in _regions():
        ref = oracle.allgather([host_u16(shard[a:min(b, SHARD)])], b - a)
        assert np.array_equal(host_u16(replica[a:b]), ref), f"replica differs in [{a}, {b})"
    idx = stratified_sample(PSI, 1 << 20, 0xB1, edge=0)
    idx_d = torch.from_numpy(idx).to(dev)
    assert np.array_equal(host_u16(replica.index_select(0, idx_d)), host_u16(shard.index_select(0, idx_d)))
    # every element, on the device, in chunks (the copy must be exact)
    step = 1 << 30
    for a in range(0, PSI, step):
        b = min(PSI, a + step)
        assert torch.equal(replica[a:b].view(torch.int16), shard[a:b].view(torch.int16)), f"chunk at {a}"
    del shard, replica
    torch.cuda.empty_cache()


@pytest.mark.timeout(900)
def test_qwz_allgather_beyond_launch_limit(dev):
    import torch
    torch.cuda.empty_cache()
    say(f"qwZ all-gather: shard {SHARD:,} codes, psi {PSI:,}")
    gen = torch.Generator(device=dev)
    gen.manual_seed(0xB2)
    codes = torch.randint(-127, 128, (SHARD,), dtype=torch.int8, device=dev, generator=gen)
    nsc = zs.qwz_scales_len(SHARD)
    scales = (torch.rand(nsc, dtype=torch.float32, device=dev, generator=gen) * 1e-3 + 1e-6)
    replica = torch.empty(PSI, dtype=torch.float16, device=dev)
    zs.qwz_allgather([codes], [scales], replica)
    torch.cuda.synchronize()
    blk = zs.ZERO_QWZ_BLOCK
    for a, b in _regions():
        # whole qwZ blocks: a is a multiple of the block size
        c = codes[a:b].cpu().numpy()
        sc = scales[a // blk:(b + blk - 1) // blk].cpu().numpy()
        ref = oracle.qwz_dequantize(c, sc)
        assert np.array_equal(host_u16(replica[a:b]), ref), f"replica differs in [{a}, {b})"
    # a stratified sample of whole blocks
    starts = (stratified_sample(PSI // blk, 4096, 0xB2, edge=0) * blk).astype(np.int64)
    for s0 in starts[::64]:
        e0 = min(PSI, s0 + blk)
        ref = oracle.qwz_dequantize(codes[s0:e0].cpu().numpy(), scales[s0 // blk:s0 // blk + 1].cpu().numpy())
        assert np.array_equal(host_u16(replica[s0:e0]), ref), f"block at {s0}"
    del codes, scales, replica
    torch.cuda.empty_cache()
