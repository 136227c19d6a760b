"""Pins for the oracle's all-gather of the fp16 shards ("ZeRO Stage 1 Math",
"The per-step mechanics" beat 4; "DeepSpeed ZeRO Stages" 3.1): the flat
replica is the concatenation of the ranks' shards in rank order without the
padding.  Checked against numpy's concatenation of the real parts, and by a
scatter/gather round trip through the partition layout."""
import numpy as np
import pytest


@pytest.mark.parametrize("psi,n,align", [(0, 3, 8), (1, 1, 1), (1000, 4, 8), (1001, 4, 8), (5000, 7, 128),
                                         (129, 64, 1), (200, 8, 128)])
def test_allgather_is_concatenation_of_real_parts(orc, psi, n, align):
    rng = np.random.default_rng(psi + n)
    L = orc.partition_layout(psi, n, 0, align)[1][2]
    shards = [rng.integers(0, 65536, L, dtype=np.uint64).astype(np.uint16) for _ in range(n)]
    reals = [orc.partition_layout(psi, n, r, align)[1][4] for r in range(n)]
    want = np.concatenate([s[:k] for s, k in zip(shards, reals)]) if psi else np.zeros(0, np.uint16)
    if L == 0:
        return
    got = orc.allgather(shards, psi)
    assert np.array_equal(got, want)


def test_scatter_gather_round_trip(orc):
    rng = np.random.default_rng(5)
    psi, n = 1_000_003, 6
    replica = rng.integers(0, 65536, psi, dtype=np.uint64).astype(np.uint16)
    shards = []
    for r in range(n):
        _, (_, _, L, off, real) = orc.partition_layout(psi, n, r, 128)
        sh = np.full(L, 0xDEAD, dtype=np.uint16)           # padding holds junk
        sh[:real] = replica[off:off + real]
        shards.append(sh)
    assert np.array_equal(orc.allgather(shards, psi), replica)
