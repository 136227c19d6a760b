#!/usr/bin/env python3
"""Benchmark of one ZeRO rank's shard optimizer step on one MI355X.

Workload (the graded one): a GPT-2-XL-scale model, psi = 1.5e9 parameters
split over N = 4 ranks with align 128; rank 0 owns a 375,000,064-parameter
shard.  fp32 master ~ N(0, 0.02), m ~ N(0, 1e-4), v ~ |N(0, 1e-6)|, one
pre-reduced fp16 gradient ~ f16(N(0, 1e-3) * 2^16), loss scale 2^16, Adam
lr 1e-4, betas (0.9, 0.999), eps 1e-8, t = 1000, 1001, ...  All inputs are
synthetic, seeded, and resident in HBM before timing starts.

One step = the whole hot path on that shard: the partition layout (host),
the gradient statistics (overflow flag + sum of squares, two kernels) and the
fused Adam update (one kernel).  ``value`` is shard parameters per second of
wall time over the K timed steps.  The algorithmic traffic is 30 bytes per
parameter for the whole call (2 for the statistics pass, 28 for the update).

Also reported: the update kernel alone against the HBM roofline (HIP events
around each launch, on the launch stream), the statistics pass timed the
same way inside the same steps, a plain copy/read kernel as the
attainable ceiling, the update with global-norm clipping, the owner-side
reduce of 64 fp16 slices of the 7.5B / N = 64 shard (117,187,584
parameters), the fp16 all-gather and the qwZ block-INT8 variants (encoder
fused into the update, encoder alone, decoding all-gather), the step on the
other workload shapes (tiny, 7.5B / N = 64, 7B / N = 8, 1.5e9 / N = 1), the CPU oracle
timed on a bounded sample of the same workload on one host core, and the
multi-core SIMD host step (ZeRO-Offload's CPU Adam) on the whole shard.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "shard Adam step: params/sec and HBM GB/s (% of peak), 1 GPU"
PEAK_HBM_GBPS = 8000.0
UPDATE_BYTES_PER_PARAM = 28      # read g2 m4 v4 th4, write m4 v4 th4 p16 2
STATS_BYTES_PER_PARAM = 2        # read g2
REDUCE_BYTES_PER_PARAM = lambda n: 2 * n + 4   # noqa: E731
QWZ_BYTES_PER_PARAM = 1 + 4 / 256               # int8 code + one fp32 scale per 256 values
COUNTERS_FILE = os.path.join(ROOT, "profiles", "adam_update_gpt2xl_shard_counters.txt")
REDUCE_COUNTERS_FILE = os.path.join(ROOT, "profiles", "grad_reduce_7p5b_n64_counters.txt")
STATS_COUNTERS_FILE = os.path.join(ROOT, "profiles", "grad_stats_gpt2xl_shard_counters.txt")
ALLGATHER_COUNTERS_FILE = os.path.join(ROOT, "profiles", "allgather_gpt2xl_counters.txt")
QWZ_COUNTERS_FILES = {k: os.path.join(ROOT, "profiles", f) for k, f in (
    ("update_fused", "adam_update_qwz_gpt2xl_shard_counters.txt"),
    ("quantize_shard", "qwz_quantize_gpt2xl_shard_counters.txt"),
    ("allgather_gpt2xl", "qwz_allgather_gpt2xl_counters.txt"))}
KERNEL_SOURCES = [os.path.join(ROOT, "zero_partitioned_mixed_flat_amd", "csrc", f)
                  for f in ("shard_kernels.hpp", "zero_shard.hip")]

PSI, N_RANKS, RANK, ALIGN = 1_500_000_000, 4, 0, 128
SEED = 0xC2
LR, BETAS, EPS, INV_SCALE, T0 = 1e-4, (0.9, 0.999), 1e-8, 2.0 ** -16, 1000


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def counter_traffic(path=COUNTERS_FILE):
    """HBM bytes per launch from a committed rocprofv3 counter summary, or
    None when it is missing or was taken for other kernel code."""
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256") != kernel_source_hash():
        return None
    try:
        return float(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def ceiling(torch, tk, dev, n_floats=1 << 30, reps=5):
    """Plain copy (8 B/element), in-place read-modify-write with the
    update's store policy (8 B/element) and read (4 B/element), GB/s."""
    from zero_partitioned_mixed_flat_amd import probes
    src = torch.ones(n_floats, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    sink = torch.empty(1 << 16, dtype=torch.float32, device=dev)
    out = {}
    for name, fn, bytes_per in (("copy", lambda: tk.copy_f32(src, dst), 8),
                                ("rmw", lambda: probes.rmw_f32(dst), 8),
                                ("read", lambda: tk.read_f32(src, sink), 4)):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        out[f"{name}_gbps"] = round(bytes_per * n_floats * reps / (a.elapsed_time(b) * 1e-3) / 1e9, 1)
    del src, dst
    return out


def reduce_secondary(torch, zs, tk, dev, steps):
    """Owner-side reduce of 64 simulated fp16 slices (7.5B model, N = 64)."""
    lay = zs.partition_layout(7_500_000_000, 64, 0, 128)
    n = lay.shard_len
    slices = [tk.normal_f16_(torch.empty(n, dtype=torch.float16, device=dev), 1e-3 * 4096, 0xC3,
                             tk.STREAM_GRAD + r) for r in range(64)]
    out = torch.empty(n, dtype=torch.float32, device=dev)
    stats = zs.new_stats(dev)
    ws = zs.new_workspace(n, dev)
    s = 2.0 ** -12 / 64
    for _ in range(2):
        zs.grad_reduce(slices, out, stats=stats, inv_grad_scale=s, workspace=ws)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        zs.grad_reduce(slices, out, stats=stats, inv_grad_scale=s, workspace=ws)
    b.record()
    torch.cuda.synchronize()
    sec = a.elapsed_time(b) * 1e-3 / steps
    gbps = REDUCE_BYTES_PER_PARAM(64) * n / sec / 1e9
    del slices
    return {"workload": "7.5B model at N=64: owner-side sum of 64 fp16 slices of a 117,187,584-param shard "
                        "into fp32 with fused flag/sum of squares",
            "ms": round(sec * 1e3, 4), "params_per_s": n / sec, "hbm_gbps": round(gbps, 1),
            "frac_of_peak": round(gbps / PEAK_HBM_GBPS, 4), "bytes_per_param": REDUCE_BYTES_PER_PARAM(64),
            "traffic": counter_traffic(REDUCE_COUNTERS_FILE)}


def allgather_secondary(torch, zs, tk, dev, steps):
    """The fp16 all-gather of the GPT-2-XL layout: four 375,000,064-value
    shards concatenated into the 1.5e9-value flat replica (4 B/param)."""
    L = zs.partition_layout(PSI, N_RANKS, 0, ALIGN).shard_len
    shards = [tk.normal_f16_(torch.empty(L, dtype=torch.float16, device=dev), 1.0, 0xA6, tk.STREAM_GRAD + r)
              for r in range(N_RANKS)]
    replica = torch.empty(PSI, dtype=torch.float16, device=dev)
    for _ in range(2):
        zs.allgather(shards, replica)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        zs.allgather(shards, replica)
    b.record()
    torch.cuda.synchronize()
    sec = a.elapsed_time(b) * 1e-3 / steps
    gbps = 4 * PSI / sec / 1e9
    del shards, replica
    return {"workload": "fp16 all-gather of the GPT-2-XL layout: 4 shards of 375,000,064 -> 1.5e9-value replica",
            "ms": round(sec * 1e3, 4), "params_per_s": PSI / sec, "hbm_gbps": round(gbps, 1),
            "frac_of_peak": round(gbps / PEAK_HBM_GBPS, 4), "bytes_per_param": 4,
            "traffic": counter_traffic(ALLGATHER_COUNTERS_FILE)}


def _avg_ms(torch, fn, steps, before=None):
    """Mean duration of `fn`'s device work, HIP events on the current stream;
    `before`, when given, runs untimed ahead of each call."""
    evs = []
    for _ in range(steps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        if before is not None:
            before()
        a.record()
        fn()
        b.record()
        evs.append((a, b))
    torch.cuda.synchronize()
    return sum(a.elapsed_time(b) for a, b in evs) / len(evs)


def qwz_secondary(torch, zs, tk, dev, steps, g, master, m, v, p16, stats, ws, t0):
    """qwZ block-INT8 weights (blocks of 256, one fp32 scale each): the update
    with the encoder fused into its write-back, the encoder alone on the fp16
    shard, and the decoding all-gather of the GPT-2-XL layout."""
    L = master.numel()
    codes = torch.empty(L, dtype=torch.int8, device=dev)
    scales = torch.empty(zs.qwz_scales_len(L), dtype=torch.float32, device=dev)
    step = [t0]

    def fused():
        zs.adam_step(g, master, m, v, p16, step=step[0], lr=LR, betas=BETAS, eps=EPS, inv_grad_scale=INV_SCALE,
                     stats=stats, stats_precomputed=True, qwz_codes=codes, qwz_scales=scales)
        step[0] += 1
    fused()
    # each fused update follows its statistics pass, as in the step
    fused_ms = _avg_ms(torch, fused, steps,
                       before=lambda: zs.grad_stats(g, stats, inv_grad_scale=INV_SCALE, workspace=ws))
    fused_bytes = UPDATE_BYTES_PER_PARAM + QWZ_BYTES_PER_PARAM
    enc = lambda: zs.qwz_quantize(p16, codes, scales)  # noqa: E731
    enc()
    enc_ms = _avg_ms(torch, enc, steps)
    enc_bytes = 2 + QWZ_BYTES_PER_PARAM
    del codes, scales
    torch.cuda.empty_cache()

    all_codes, all_scales = [], []
    for r in range(N_RANKS):
        x = tk.normal_f16_(torch.empty(L, dtype=torch.float16, device=dev), 0.02, 0xA7, tk.STREAM_MASTER + r)
        all_codes.append(torch.empty(L, dtype=torch.int8, device=dev))
        all_scales.append(torch.empty(zs.qwz_scales_len(L), dtype=torch.float32, device=dev))
        zs.qwz_quantize(x, all_codes[-1], all_scales[-1])
        del x
    replica = torch.empty(PSI, dtype=torch.float16, device=dev)
    gat = lambda: zs.qwz_allgather(all_codes, all_scales, replica)  # noqa: E731
    gat()
    gat_ms = _avg_ms(torch, gat, steps)
    gat_bytes = QWZ_BYTES_PER_PARAM + 2
    del all_codes, all_scales, replica
    torch.cuda.empty_cache()

    def entry(key, workload, ms, n, bytes_per):
        gbps = bytes_per * n / (ms * 1e-3) / 1e9
        return {"workload": workload, "avg_launch_ms": round(ms, 4), "params_per_s": n / (ms * 1e-3),
                "hbm_gbps": round(gbps, 1), "frac_of_peak": round(gbps / PEAK_HBM_GBPS, 4),
                "bytes_per_param": bytes_per, "traffic": counter_traffic(QWZ_COUNTERS_FILES[key])}
    return {
        "update_fused": entry("update_fused", "GPT-2-XL shard update with qwZ encoding of the fresh fp16 weights",
                              fused_ms, L, fused_bytes),
        "quantize_shard": entry("quantize_shard", "qwZ encoding of the 375,000,064-value fp16 shard", enc_ms, L,
                                enc_bytes),
        "allgather_gpt2xl": entry("allgather_gpt2xl", "qwZ all-gather of the GPT-2-XL layout: 4 encoded shards -> "
                                  "1.5e9-value fp16 replica", gat_ms, PSI, gat_bytes),
    }


def _median_ms(torch, fn, steps):
    evs = []
    for _ in range(steps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        evs.append((a, b))
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in evs)
    return (ms[(len(ms) - 1) // 2] + ms[len(ms) // 2]) / 2, ms[0]


def other_configs_secondary(torch, zs, tk, dev, steps):
    """The step on the other workload shapes: the tiny one (reduce of 4
    slices + update with the fp32 sum; launch-bound, cache-resident), the
    7.5B / N = 64 shard (reduce of 64 slices + update with the fp32 sum), the
    7B / N = 8 shard and the unpartitioned 1.5e9 model (statistics + update
    with the fp16 gradient).  Median and minimum of `steps` timed steps."""
    out = {}

    def entry(workload, n, bytes_per, fn, t0):
        t = [t0]

        def run():
            fn(t[0])
            t[0] += 1
        for _ in range(3):
            run()
        med, mn = _median_ms(torch, run, steps)
        gbps = bytes_per * n / (med * 1e-3) / 1e9
        return {"workload": workload, "shard_len": n, "median_ms": round(med, 4), "min_ms": round(mn, 4),
                "params_per_s": n / (med * 1e-3), "bytes_per_param": bytes_per, "hbm_gbps": round(gbps, 1),
                "frac_of_peak": round(gbps / PEAK_HBM_GBPS, 4)}

    def reduce_step(psi, n_ranks, seed, slice_scale, s, t0, name):
        n = zs.partition_layout(psi, n_ranks, 0, 128).shard_len
        slices = [tk.normal_f16_(torch.empty(n, dtype=torch.float16, device=dev), slice_scale, seed,
                                 tk.STREAM_GRAD + r) for r in range(n_ranks)]
        master, m, v, p16 = tk.init_shard_state(n, seed, zero_moments=(t0 == 1), device=dev)
        gsum = torch.empty(n, dtype=torch.float32, device=dev)
        stats, ws = zs.new_stats(dev), zs.new_workspace(n, dev)

        def fn(t):
            zs.grad_reduce(slices, gsum, stats=stats, inv_grad_scale=s, workspace=ws)
            zs.adam_step(gsum, master, m, v, p16, step=t, lr=LR, betas=BETAS, eps=EPS, inv_grad_scale=s,
                         stats=stats, stats_precomputed=True)
        res = entry(name, n, REDUCE_BYTES_PER_PARAM(n_ranks) + 30, fn, t0)
        if n < (1 << 22):
            # launch-bound: the same calls captured once in a HIP graph and
            # replayed (the step number is fixed in the captured launch)
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                fn(t0 + 100)
            for _ in range(3):
                graph.replay()
            med, mn = _median_ms(torch, graph.replay, steps)
            res["graph_replay_median_ms"], res["graph_replay_min_ms"] = round(med, 4), round(mn, 4)
            del graph
        del slices, master, m, v, p16, gsum
        torch.cuda.empty_cache()
        return res

    def stats_step(psi, n_ranks, seed, t0, name, student=False):
        n = zs.partition_layout(psi, n_ranks, 0, 128).shard_len
        master, m, v, p16 = tk.init_shard_state(n, seed, zero_moments=student, device=dev)
        g = torch.empty(n, dtype=torch.float16, device=dev)
        if student:
            tk.student_t3_f16_(g, 1e-3 * 65536, seed, tk.STREAM_GRAD, redraw_overflow=True)
        else:
            tk.normal_f16_(g, 1e-3 * 65536, seed, tk.STREAM_GRAD)
        stats, ws = zs.new_stats(dev), zs.new_workspace(n, dev)

        def fn(t):
            zs.grad_stats(g, stats, inv_grad_scale=INV_SCALE, workspace=ws)
            zs.adam_step(g, master, m, v, p16, step=t, lr=LR, betas=BETAS, eps=EPS, inv_grad_scale=INV_SCALE,
                         stats=stats, stats_precomputed=True)
        res = entry(name, n, UPDATE_BYTES_PER_PARAM + STATS_BYTES_PER_PARAM, fn, t0)
        del master, m, v, p16, g
        torch.cuda.empty_cache()
        return res

    out["tiny_n4"] = reduce_step(1_048_576, 4, 0xC1, 1e-3 * 65536, 2.0 ** -18, 1,
                                 "tiny: psi=1,048,576, N=4, reduce of 4 slices + update (fp32 sum); "
                                 "launch-bound and cache-resident, not a roofline figure")
    out["7p5b_n64"] = reduce_step(7_500_000_000, 64, 0xC3, 1e-3 * 4096, 2.0 ** -18, 10,
                                  "7.5B at N=64: reduce of 64 slices + update (fp32 sum)")
    out["7b_n8"] = stats_step(7_000_000_000, 8, 0xC4, 1000, "7B at N=8: statistics + update (fp16 grad)")
    out["1p5b_n1"] = stats_step(1_500_000_000, 1, 0xC5, 1,
                                "GPT-2-XL unpartitioned (N=1): statistics + update (fp16 Student-t(3) grad, "
                                "overflowing draws redrawn)", student=True)
    return out


def cpu_baseline(torch, g, master, m, v, p16, target_s=10.0):
    """The oracle (single-threaded C, untuned) on the first 2^24 parameters of
    the shard: statistics then the gated update, repeated until ~10 s."""
    import numpy as np
    import oracle
    n = 1 << 24
    g_h = g[:n].cpu().view(torch.int16).numpy().view(np.uint16).copy()
    st = [master[:n].cpu().numpy().copy(), m[:n].cpu().numpy().copy(), v[:n].cpu().numpy().copy(),
          p16[:n].cpu().view(torch.int16).numpy().view(np.uint16).copy()]
    # the oracle is single-threaded: pin it to one host core while it runs
    pinned = None
    if hasattr(os, "sched_getaffinity"):
        allowed = os.sched_getaffinity(0)
        pinned = min(allowed)
        os.sched_setaffinity(0, {pinned})
    try:
        reps = 0
        t0 = time.perf_counter()
        while True:
            rc, _, _ = oracle.shard_adam_step(g_h, *st, step=T0 + reps, lr=LR, beta1=BETAS[0], beta2=BETAS[1],
                                              eps=EPS, inv_scale=INV_SCALE)
            assert rc == 0
            reps += 1
            el = time.perf_counter() - t0
            if el >= target_s:
                break
    finally:
        if pinned is not None:
            os.sched_setaffinity(0, allowed)
    cpu_model = platform.processor() or "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    rate = n * reps / el
    return {"value": rate, "unit": "params/s", "cores": 1, "kind": "oracle",
            "sample": f"first {n:,} params of the 375,000,064-param shard, statistics + update, "
                      f"{reps} repetitions in {el:.1f} s",
            "gbps": round(rate * (UPDATE_BYTES_PER_PARAM + STATS_BYTES_PER_PARAM) / 1e9, 2),
            "pinned_core": pinned, "host_cpu": cpu_model, "host_threads": os.cpu_count()}


def host_adam_secondary(torch, g, master, m, v, p16, steps=3):
    """The multi-core SIMD host step (ZeRO-Offload's CPU Adam) on the whole
    shard in host memory: statistics + update, all OpenMP threads."""
    import numpy as np

    from zero_partitioned_mixed_flat_amd import host_adam as ha
    n = master.numel()
    g_h = g.cpu().view(torch.int16).numpy().view(np.uint16).copy()
    st = [master.cpu().numpy().copy(), m.cpu().numpy().copy(), v.cpu().numpy().copy(),
          p16.cpu().view(torch.int16).numpy().view(np.uint16).copy()]
    threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or (os.cpu_count() or 1)
    isa = ha.set_isa(0)
    ha.adam_step(g_h, *st, step=T0, lr=LR, betas=BETAS, eps=EPS, inv_grad_scale=INV_SCALE, threads=threads)
    t0 = time.perf_counter()
    for k in range(steps):
        ha.adam_step(g_h, *st, step=T0 + 1 + k, lr=LR, betas=BETAS, eps=EPS, inv_grad_scale=INV_SCALE,
                     threads=threads)
    el = (time.perf_counter() - t0) / steps
    return {"value": n / el, "unit": "params/s", "cores": threads, "kind": "host SIMD+OpenMP step",
            "isa": ha.ISA_NAMES[isa], "ms_per_step": round(el * 1e3, 2),
            "host_gbps": round((UPDATE_BYTES_PER_PARAM + STATS_BYTES_PER_PARAM) * n / el / 1e9, 1),
            "sample": f"the whole {n:,}-param shard in host memory, statistics + update, {steps} timed steps"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-other-configs", action="store_true",
                    help="skip the other workload shapes (profiling runs: keeps one shape per kernel)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one rank's shard step on one GPU and supports --gpus 1 only: each "
              "rank's step is independent of the others, so the per-rank throughput is the one-GPU "
              "figure; the multi-GPU exchange is not implemented.", file=sys.stderr)
        sys.exit(2)

    import torch
    import zero_partitioned_mixed_flat_amd as zs
    from zero_partitioned_mixed_flat_amd import testkit as tk

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    lay = zs.partition_layout(PSI, N_RANKS, RANK, ALIGN)
    L = lay.shard_len
    log(f"workload: psi={PSI} N={N_RANKS} rank={RANK} shard_len={L}")
    master, m, v, p16 = tk.init_shard_state(L, SEED, zero_moments=False, device=dev)
    g = tk.normal_f16_(torch.empty(L, dtype=torch.float16, device=dev), 1e-3 * 65536, SEED, tk.STREAM_GRAD)
    stats = zs.new_stats(dev)
    ws = zs.new_workspace(L, dev)
    torch.cuda.synchronize()

    ceil = ceiling(torch, tk, dev)
    log(f"ceiling: {ceil}")

    def one_step(t, ev=None):
        layout = zs.partition_layout(PSI, N_RANKS, RANK, ALIGN)          # a1 (host)
        assert layout.shard_len == L
        if ev is not None:
            ev[2].record()
        zs.grad_stats(g, stats, inv_grad_scale=INV_SCALE, workspace=ws)  # a3 (2 kernels)
        if ev is not None:
            ev[0].record()
        zs.adam_step(g, master, m, v, p16, step=t, lr=LR, betas=BETAS, eps=EPS, inv_grad_scale=INV_SCALE,
                     stats=stats, stats_precomputed=True)                # a4-a8 (1 kernel)
        if ev is not None:
            ev[1].record()

    for i in range(args.warmup):
        one_step(T0 + i)
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} steps done; flag/sumsq = {zs.read_stats(stats)}")

    evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for k in range(args.steps):
        one_step(T0 + args.warmup + k, evs[k])
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    dev_s = start.elapsed_time(end) * 1e-3
    upd_ms = [e[0].elapsed_time(e[1]) for e in evs]
    stats_ms = [e[2].elapsed_time(e[0]) for e in evs]     # statistics + finalize
    stats_avg_s = sum(stats_ms) / len(stats_ms) * 1e-3
    upd_avg_s = sum(upd_ms) / len(upd_ms) * 1e-3
    upd_sorted = sorted(upd_ms)
    upd_median_ms = (upd_sorted[(len(upd_ms) - 1) // 2] + upd_sorted[len(upd_ms) // 2]) / 2
    overflow, sumsq = zs.read_stats(stats)
    log(f"timed {args.steps} steps: wall {wall * 1e3:.3f} ms, device {dev_s * 1e3:.3f} ms, "
        f"update avg {upd_avg_s * 1e3:.4f} ms, overflow={overflow}")

    step_s = wall / args.steps
    value = L / step_s
    whole_gbps = (UPDATE_BYTES_PER_PARAM + STATS_BYTES_PER_PARAM) * L / step_s / 1e9
    upd_gbps = UPDATE_BYTES_PER_PARAM * L / upd_avg_s / 1e9
    traffic = counter_traffic()
    stats_traffic = counter_traffic(STATS_COUNTERS_FILE)
    # HBM bytes of the whole step from the counters (statistics + update; the
    # 16-byte finalize is negligible), over the wall time of a step
    step_counter_bytes = traffic + stats_traffic if traffic is not None and stats_traffic is not None else None

    secondary = None
    if not args.no_secondary:
        # the same update with global-norm clipping active (max norm 1; this
        # gradient's norm is about 19): the factor comes from the device sum
        # of squares, so the kernel's traffic is unchanged.  Each update
        # follows its own statistics pass, as in the step, so that it finds
        # the gradient's tail in the Infinity Cache like the timed update.
        clip_ms = []
        for k in range(args.steps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            zs.grad_stats(g, stats, inv_grad_scale=INV_SCALE, workspace=ws)
            a.record()
            zs.adam_step(g, master, m, v, p16, step=T0 + 100 + k, lr=LR, betas=BETAS, eps=EPS,
                         inv_grad_scale=INV_SCALE, max_grad_norm=1.0, stats=stats, stats_precomputed=True)
            b.record()
            clip_ms.append((a, b))
        torch.cuda.synchronize()
        clip_avg = sum(a.elapsed_time(b) for a, b in clip_ms) / len(clip_ms)
        zs.grad_stats(g, stats, inv_grad_scale=INV_SCALE, workspace=ws)
        qwz = qwz_secondary(torch, zs, tk, dev, args.steps, g, master, m, v, p16, stats, ws, T0 + 200)
        del ws
        secondary = {"clipped_update": {"max_grad_norm": 1.0, "avg_launch_ms": round(clip_avg, 4),
                                        "hbm_gbps": round(UPDATE_BYTES_PER_PARAM * L / (clip_avg * 1e-3) / 1e9, 1)},
                     "qwz": qwz,
                     "reduce_n64": reduce_secondary(torch, zs, tk, dev, max(5, args.steps // 2)),
                     "allgather_gpt2xl": allgather_secondary(torch, zs, tk, dev, max(5, args.steps // 2))}
        if not args.no_other_configs:
            secondary["other_configs"] = other_configs_secondary(torch, zs, tk, dev, max(5, args.steps // 2))
        log(f"secondary: {secondary}")

    cpu = None
    host = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(torch, g, master, m, v, p16)
        cpu["gpu_over_oracle"] = round(value / cpu["value"], 1)
        log(f"cpu baseline: {cpu}")
        host = host_adam_secondary(torch, g, master, m, v, p16)
        log(f"host SIMD step: {host}")

    rec = {
        "metric": METRIC, "value": value, "unit": "params/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(step_s * 1e3, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "GPT-2-XL-scale shard: psi=1.5e9, N=4, rank 0 owns 375,000,064 params "
                               "(align 128); fp16 grad N(0,1e-3)*2^16, fp32 master N(0,0.02), m N(0,1e-4), "
                               "v |N(0,1e-6)|, Adam lr 1e-4 betas (0.9,0.999) eps 1e-8, t from 1000",
                   "psi": PSI, "n_ranks": N_RANKS, "shard_len": L, "grad_dtype": "f16",
                   "algorithmic_bytes_per_param": UPDATE_BYTES_PER_PARAM + STATS_BYTES_PER_PARAM},
        "hbm_gbps": round(whole_gbps, 1), "hbm_frac_of_peak": round(whole_gbps / PEAK_HBM_GBPS, 4),
        "hbm_gbps_counters": (round(step_counter_bytes / step_s / 1e9, 1) if step_counter_bytes else None),
        "update_params_per_s": L / (upd_median_ms * 1e-3),
        "roofline": {"kernel": "adam_update_kernel<f16>", "bound": "hbm", "achieved": round(upd_gbps, 1),
                     "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": round(upd_gbps / PEAK_HBM_GBPS, 4),
                     "traffic": traffic, "avg_launch_ms": round(upd_avg_s * 1e3, 4),
                     "median_launch_ms": round(upd_median_ms, 4), "min_launch_ms": round(upd_sorted[0], 4),
                     "algorithmic_bytes_per_launch": UPDATE_BYTES_PER_PARAM * L,
                     # the same-box ceiling of an in-place read-modify-write stream
                     # (measured in this run), which cancels box-to-box spread
                     "rmw_ceiling_gbps": ceil.get("rmw_gbps"),
                     "frac_of_rmw_ceiling": (round(upd_gbps / ceil["rmw_gbps"], 4) if ceil.get("rmw_gbps")
                                             else None)},
        "statistics": {"kernels": "grad_stats_kernel<f16> + finalize_stats_kernel", "bound": "hbm",
                       "avg_ms": round(stats_avg_s * 1e3, 4),
                       "achieved": round(STATS_BYTES_PER_PARAM * L / stats_avg_s / 1e9, 1), "unit": "GB/s",
                       "frac": round(STATS_BYTES_PER_PARAM * L / stats_avg_s / 1e9 / PEAK_HBM_GBPS, 4),
                       "traffic": stats_traffic, "algorithmic_bytes_per_launch": STATS_BYTES_PER_PARAM * L},
        "ceiling": ceil,
        "secondary": secondary,
        "cpu_baseline": cpu,
        "host_adam": host,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
