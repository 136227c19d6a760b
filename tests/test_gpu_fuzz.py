"""Seeded random combinations of the path's options against the oracle.
Each case draws a length (log-uniform from 1 to 2M, or just around a tile
size), a gradient source (the reduce of 1..64 fp16 slices into fp32, an
fp16 gradient with the statistics formed inside the step or beforehand, or
an fp32 gradient), qwZ encoding on or off, global-norm clipping on or off
(with a bound around the gradient's norm, so that some cases clip and some
do not), the step number, the gradient scale, zero or random moments, and
now and then one non-finite gradient entry.  The reduce's sum, the flag and
every state array and qwZ output must equal the oracle's bit for bit; the
sum of squares agrees to a relative 1e-10."""
import numpy as np
import pytest

import oracle
import zero_partitioned_mixed_flat_amd as zs
from zero_partitioned_mixed_flat_amd import testkit as tk
from gpu_util import assert_state_parity, assert_stats, host_f32, host_u16, require_gpu, say

pytestmark = pytest.mark.gpu

LR, BETAS, EPS = 1e-4, (0.9, 0.999), 1e-8
CASES = 48


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def _cases():
    rng = np.random.default_rng(0xF022)
    out = []
    for i in range(CASES):
        if rng.random() < 0.25:
            n = int(rng.choice([256, 512, 1024, 2048, 4096, 8192, 16384, 32768])) + int(rng.integers(-3, 4))
        else:
            n = int(np.exp(rng.uniform(0.0, np.log(2_000_000))))
        n = max(n, 1)
        source = str(rng.choice(["reduce", "f16_inside", "f16_before", "f32"]))
        n_slices = int(rng.choice([1, 2, 3, 4, 8, 17, 64])) if source == "reduce" else 1
        n_slices = max(1, min(n_slices, 40_000_000 // n))
        out.append(dict(
            case=i, n=n, source=source, n_slices=n_slices, qwz=bool(rng.random() < 0.4),
            clip=bool(rng.random() < 0.4), clip_rel=float(rng.uniform(0.3, 2.0)),
            step=int(rng.choice([1, 2, 3, 10, 1000, int(rng.integers(1, 10**6))])),
            scale_pow=int(rng.integers(10, 21)), zero_moments=bool(rng.random() < 0.5),
            special=str(rng.choice(["none"] * 6 + ["inf", "-inf", "nan"])),
            special_pos=float(rng.random()), seed=0xF000 + i))
    return out


@pytest.mark.parametrize("c", _cases(), ids=lambda c: f"case{c['case']}-{c['source']}-n{c['n']}")
def test_random_configuration_matches_oracle(dev, c):
    import torch
    n, s = c["n"], 2.0 ** -c["scale_pow"]
    say(f"fuzz {c}")
    master, m, v, p16 = tk.init_shard_state(n, c["seed"], zero_moments=c["zero_moments"], device=dev)
    ref = [host_f32(master), host_f32(m), host_f32(v), host_u16(p16)]
    pos = min(n - 1, int(c["special_pos"] * n))
    special = {"inf": float("inf"), "-inf": float("-inf"), "nan": float("nan")}.get(c["special"])
    stats, ws = zs.new_stats(dev), zs.new_workspace(n, dev)

    # the gradient the update sees, on the device and as the oracle's input
    precomputed = True
    if c["source"] == "reduce":
        slices = [tk.normal_f16_(torch.empty(n, dtype=torch.float16, device=dev), 1e-3 * 2 ** c["scale_pow"],
                                 c["seed"], tk.STREAM_GRAD + r) for r in range(c["n_slices"])]
        if special is not None:
            slices[-1][pos] = special
        g = torch.empty(n, dtype=torch.float32, device=dev)
        s = s / c["n_slices"]
        zs.grad_reduce(slices, g, stats=stats, inv_grad_scale=s, workspace=ws)
        g_ref = oracle.grad_reduce([host_u16(t) for t in slices])
        got_sum = host_f32(g)
        assert np.array_equal(got_sum.view(np.uint32), g_ref.view(np.uint32)), "reduce sum differs"
    elif c["source"] == "f32":
        g = tk.normal_f32_(torch.empty(n, dtype=torch.float32, device=dev), 0.0, 1e-3 / s, c["seed"],
                           tk.STREAM_GRAD)
        if special is not None:
            g[pos] = special
        g_ref = host_f32(g)
        zs.grad_stats(g, stats, inv_grad_scale=s, workspace=ws)
    else:
        g = tk.normal_f16_(torch.empty(n, dtype=torch.float16, device=dev), 1e-3 * 2 ** c["scale_pow"], c["seed"],
                           tk.STREAM_GRAD)
        if special is not None:
            g[pos] = special
        g_ref = host_u16(g)
        if c["source"] == "f16_before":
            zs.grad_stats(g, stats, inv_grad_scale=s, workspace=ws)
        else:
            precomputed = False

    flag, ssq = oracle.grad_stats(g_ref, s)
    assert flag == (0 if special is None else 1)
    max_norm = 0.0
    if c["clip"] and not flag:
        max_norm = c["clip_rel"] * float(np.sqrt(ssq))
    codes = torch.empty(n, dtype=torch.int8, device=dev) if c["qwz"] else None
    scales = torch.empty(zs.qwz_scales_len(n), dtype=torch.float32, device=dev) if c["qwz"] else None
    if c["qwz"]:
        codes.fill_(0x55)
        scales.fill_(-1.0)
    zs.adam_step(g, master, m, v, p16, step=c["step"], lr=LR, betas=BETAS, eps=EPS, inv_grad_scale=s,
                 max_grad_norm=max_norm, stats=stats, stats_precomputed=precomputed,
                 workspace=None if precomputed else ws, qwz_codes=codes, qwz_scales=scales)

    rc, rflag, rssq = oracle.shard_adam_step(g_ref, *ref, step=c["step"], lr=LR, beta1=BETAS[0],
                                             beta2=BETAS[1], eps=EPS, inv_scale=s, max_norm=max_norm)
    assert rc == 0 and rflag == flag
    assert_stats(zs.read_stats(stats), (rflag, rssq), f"case {c['case']}")
    counts = assert_state_parity([host_f32(master), host_f32(m), host_f32(v), host_u16(p16)], ref,
                                 f"case {c['case']}")
    assert sum(counts.values()) == 0, counts
    if c["qwz"]:
        if rflag:
            # a skipped step writes no codes and no scales
            assert (codes.cpu().numpy() == 0x55).all()
            assert (scales.cpu().numpy() == -1.0).all()
        else:
            rc_codes, rc_scales = oracle.qwz_quantize(ref[3])
            assert np.array_equal(codes.cpu().numpy(), rc_codes)
            assert np.array_equal(scales.cpu().numpy().view(np.uint32), rc_scales.view(np.uint32))


def _gather_cases():
    rng = np.random.default_rng(0xF033)
    out = []
    for i in range(24):
        n_ranks = int(rng.choice([1, 2, 3, 4, 7, 8, 16, 33, 64]))
        align = int(2 ** rng.integers(3, 10))      # the gathers take shard lengths in multiples of 8
        psi = max(1, int(np.exp(rng.uniform(0.0, np.log(4_000_000)))))
        out.append(dict(case=i, psi=psi, n_ranks=n_ranks, align=align, qwz=bool(rng.random() < 0.5),
                        seed=0xF100 + i))
    return out


@pytest.mark.parametrize("c", _gather_cases(),
                         ids=lambda c: f"case{c['case']}-psi{c['psi']}-N{c['n_ranks']}-a{c['align']}")
def test_random_gather_matches_oracle(dev, c):
    """The fp16 or the qwZ-decoding all-gather of a random layout (psi, N,
    align from 8 to 512): ragged last shards and padding-only shards."""
    import torch
    lay = zs.partition_layout(c["psi"], c["n_ranks"], 0, c["align"])
    L = lay.shard_len
    say(f"gather fuzz {c}, shard_len={L}")
    xs = [tk.normal_f16_(torch.empty(L, dtype=torch.float16, device=dev), 0.02, c["seed"], tk.STREAM_MASTER + r)
          for r in range(c["n_ranks"])]
    replica = torch.empty(c["psi"], dtype=torch.float16, device=dev)
    if not c["qwz"]:
        zs.allgather(xs, replica)
        want = oracle.allgather([host_u16(t) for t in xs], c["psi"])
    else:
        codes, scales, dec = [], [], []
        for x in xs:
            rc_codes, rc_scales = oracle.qwz_quantize(host_u16(x))
            codes.append(torch.from_numpy(rc_codes).to(dev))
            scales.append(torch.from_numpy(rc_scales).to(dev))
            dec.append(oracle.qwz_dequantize(rc_codes, rc_scales))
        zs.qwz_allgather(codes, scales, replica)
        want = oracle.allgather(dec, c["psi"])
    assert np.array_equal(host_u16(replica), want)
