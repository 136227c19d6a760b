"""Pins for the oracle's partition layout and model-state memory formulas.

Layout: the partition properties of "DeepSpeed ZeRO Stages" section 2
(disjoint sets, union is every index, sizes about Psi/N, rank i owns P_i) are
checked by brute force, independent of how the oracle computes the layout.
Memory: every worked figure the four pages print (tests/golden/memory_figures.txt).
"""
import math
import os

import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "memory_figures.txt")


def _check_partition(orc, psi, n, align):
    lays = []
    for r in range(n):
        st, lay = orc.partition_layout(psi, n, r, align)
        assert st == 0
        lays.append(lay)
    L = lays[0][2]
    covered = 0
    prev_end = 0
    for r, (p, ppad, shard, off, real) in enumerate(lays):
        assert p == psi and shard == L and ppad == n * L
        assert L % align == 0
        # contiguous, in rank order, no gaps and no overlaps
        assert off == prev_end
        prev_end = off + shard
        # the real (unpadded) part is the intersection with [0, psi)
        assert real == max(0, min(psi, off + shard) - off)
        covered += real
    assert covered == psi                       # union is all of {0..psi-1}
    assert prev_end == n * L >= psi
    # |P_i| about psi/N: no shard is shorter than ceil(psi/N) and padding is
    # less than one alignment unit per rank
    ceil_share = -(-psi // n)
    assert ceil_share <= L < ceil_share + align or (psi == 0 and L == 0)


@pytest.mark.parametrize("align", [1, 2, 4, 8, 16, 32, 64, 128])
def test_partition_brute_force(orc, align):
    psis = list(range(0, 300)) + list(range(300, 2001, 37)) + [1999, 2000]
    for psi in psis:
        for n in range(1, 18):
            _check_partition(orc, psi, n, align)


def test_partition_indices_disjoint_cover_small(orc):
    # explicit index sets for tiny cases: every index owned by exactly one rank
    for psi in range(0, 40):
        for n in range(1, 7):
            for align in (1, 2, 4, 8):
                owner = [0] * psi
                for r in range(n):
                    _, (_, _, shard, off, real) = orc.partition_layout(psi, n, r, align)
                    for j in range(off, off + real):
                        owner[j] += 1
                assert owner == [1] * psi


@pytest.mark.parametrize("psi,n,rank,shard,real", [
    (1_048_576, 4, 0, 262_144, 262_144),              # tiny workload, rank 0
    (1_500_000_000, 4, 0, 375_000_064, 375_000_064),  # GPT-2-XL shard
    (1_500_000_000, 4, 3, 375_000_064, 374_999_808),
    (7_500_000_000, 64, 0, 117_187_584, 117_187_584),  # 7.5B at N=64
    (7_500_000_000, 64, 63, 117_187_584, 117_182_208),
    (7_000_000_000, 8, 0, 875_000_064, 875_000_064),  # 7B at N=8
    (7_000_000_000, 8, 7, 875_000_064, 874_999_552),
    (1_500_000_000, 1, 0, 1_500_000_000, 1_500_000_000),  # unpartitioned
])
def test_partition_workload_shards(orc, psi, n, rank, shard, real):
    st, lay = orc.partition_layout(psi, n, rank, 128)
    assert st == 0
    assert lay[2] == shard and lay[4] == real
    assert lay[3] == rank * shard


def test_partition_errors(orc):
    assert orc.partition_layout(10, 0, 0, 1)[0] == -1      # N < 1
    assert orc.partition_layout(10, 4, 4, 1)[0] == -1      # rank out of range
    assert orc.partition_layout(10, 4, -1, 1)[0] == -1
    assert orc.partition_layout(10, 4, 0, 3)[0] == -1      # align not a power of 2
    assert orc.partition_layout(10, 4, 0, 0)[0] == -1
    assert orc.partition_layout(-1, 4, 0, 1)[0] == -1      # negative psi
    assert orc.partition_layout(2**62, 4, 0, 2**61)[0] == -5  # N*align overflows
    assert orc.partition_layout(2**63 - 1, 3, 0, 2**60)[0] == -5


def _golden_rows():
    rows = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            data, src = line.split("|", 1)
            psi, n, stage, K, gb, tol = data.split()
            rows.append((float(psi), int(n), int(stage), float(K), float(gb), float(tol), src.strip()))
    return rows


@pytest.mark.parametrize("row", _golden_rows(), ids=lambda r: r[6][:48])
def test_memory_figures_from_pages(orc, row):
    psi, n, stage, K, gb, tol, src = row
    got = orc.model_state_bytes(psi, n, stage, K) / 1e9
    assert abs(got - gb) <= tol + 1e-9 * gb, (src, got, gb)


def test_memory_component_figures(orc):
    # [ZS] 1.2: the fp16 compute copy of a 1.5B model is 3 GB, 2 bytes/param,
    # one eighth of the 16-byte total.
    full = orc.model_state_bytes(1.5e9, 1, 0, 12.0)
    assert math.isclose(full, 24e9) and math.isclose(full / 8, 3e9)
    # [ZS] 5.1 and section 9: offloaded Adam states need K*Psi = 84 GB for 7B.
    assert math.isclose(orc.model_state_bytes(7e9, 1, 0, 12.0) - orc.model_state_bytes(7e9, 1, 0, 0.0), 84e9)
    # [ZOS] Stage 1 discussion: the optimizer part for 7B at 64 GPUs is
    # "about 1.31 GB" (stage-1 total minus the 4 Psi replica).
    opt = orc.model_state_bytes(7e9, 64, 1, 12.0) - 4 * 7e9
    assert abs(opt / 1e9 - 1.31) < 0.005
    # [ZOS] Stage 2: the replica part is 14 GB for 7B; the page's sharded part
    # (printed as 0.9 GB) disagrees with its own (2Psi+12Psi)/N formula, which
    # the oracle follows: 14 Psi / 64 = 1.53125 GB.
    part = orc.model_state_bytes(7e9, 64, 2, 12.0) - 14e9
    assert math.isclose(part, 1.53125e9) and abs(part / 1e9 - 0.9) > 0.5
    # [S1M]: the stage-1 floor as N grows is 4 Psi = 30 GB for 7.5B
    assert abs(orc.model_state_bytes(7.5e9, 1 << 30, 1, 12.0) / 1e9 - 30.0) < 1e-6
    # [S1M] "The memory math": at N = 1 stage 1 returns the 16 Psi total
    for stage in (1, 2, 3):
        assert math.isclose(orc.model_state_bytes(7.5e9, 1, stage, 12.0), 120e9)


def test_memory_errors(orc):
    assert orc.model_state_bytes(1e9, 0, 1, 12.0) < 0
    assert orc.model_state_bytes(1e9, 4, 4, 12.0) < 0
    assert orc.model_state_bytes(-1.0, 4, 1, 12.0) < 0
