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
The steps take their gradients from three pre-generated buffers in turn, so
that no step can find an earlier step's gradient in the caches (a real step
sees a fresh gradient); the same loop over one reused buffer is reported
beside it.

Also reported: the update kernel alone against the HBM roofline (HIP events
around each launch, on the launch stream), the statistics pass timed the
same way inside the same steps, a plain copy/read kernel as the
attainable ceiling, the update with global-norm clipping, the owner-side
reduce of 64 fp16 slices of the 7.5B / N = 64 shard (117,187,584
parameters), the fp16 all-gather and the qwZ block-INT8 variants (encoder
fused into the update, encoder alone, decoding all-gather), the step on the
other workload shapes (tiny, 7.5B / N = 64, 7B / N = 8 with its skipped
step, 1.5e9 / N = 1), the CPU oracle timed on bounded samples of these
workloads on one host core, and the multi-core SIMD host step
(ZeRO-Offload's CPU Adam) on the whole shard.
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
N_GRAD_BUFFERS = 3
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
    # the access pattern's own ceilings, on the same 64 slice allocations:
    # a plain read of all slices (128 B/param), and the same read plus a
    # 4-byte output per element (132 B/param, the reduce's traffic)
    sink = torch.zeros(1024, dtype=torch.int32, device=dev)
    xout = torch.empty(n, dtype=torch.int32, device=dev)
    ceil = {}
    for name, fn, bytes_per in (("read64", lambda: tk.read_slices(slices, sink), 2 * 64),
                                ("read64_write", lambda: tk.read_slices(slices, sink, xout), 2 * 64 + 4)):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        cs = e0.elapsed_time(e1) * 1e-3 / steps
        ceil[name] = {"ms": round(cs * 1e3, 4), "gbps": round(bytes_per * n / cs / 1e9, 1)}
    del slices, xout
    return {"workload": "7.5B model at N=64: owner-side sum of 64 fp16 slices of a 117,187,584-param shard "
                        "into fp32 with fused flag/sum of squares",
            "ms": round(sec * 1e3, 4), "params_per_s": n / sec, "hbm_gbps": round(gbps, 1),
            "frac_of_peak": round(gbps / PEAK_HBM_GBPS, 4), "bytes_per_param": REDUCE_BYTES_PER_PARAM(64),
            "traffic": counter_traffic(REDUCE_COUNTERS_FILE),
            "ceiling_64_slices": ceil,
            # time of the pattern's ceilings over the reduce's time (1.0 = the
            # reduce runs as fast as plain streaming of the same slices)
            "frac_of_read64_write_ceiling": round(ceil["read64_write"]["ms"] / (sec * 1e3), 4),
            "frac_of_read64_ceiling_time": round(ceil["read64"]["ms"] / (sec * 1e3), 4)}


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


def qwz_secondary(torch, zs, tk, dev, steps, grads, master, m, v, p16, stats, ws, t0):
    """qwZ block-INT8 weights (blocks of 256, one fp32 scale each): the update
    with the encoder fused into its write-back, the encoder alone on the fp16
    shard, and the decoding all-gather of the GPT-2-XL layout."""
    L = master.numel()
    codes = torch.empty(L, dtype=torch.int8, device=dev)
    scales = torch.empty(zs.qwz_scales_len(L), dtype=torch.float32, device=dev)
    step = [t0]

    def fused():
        g = grads[step[0] % len(grads)]
        zs.adam_step(g, master, m, v, p16, step=step[0], lr=LR, betas=BETAS, eps=EPS, inv_grad_scale=INV_SCALE,
                     stats=stats, stats_precomputed=True, qwz_codes=codes, qwz_scales=scales)
        step[0] += 1

    def before():
        zs.grad_stats(grads[step[0] % len(grads)], stats, inv_grad_scale=INV_SCALE, workspace=ws)
    before()
    fused()
    # each fused update follows its statistics pass, as in the step
    fused_ms = _avg_ms(torch, fused, steps, before=before)
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
    7B / N = 8 shard (statistics + update with the fp16 gradient, and the
    same step on a gradient holding +inf, which is skipped) and the
    unpartitioned 1.5e9 model.  Median and minimum of `steps` timed steps;
    the statistics-based steps take their gradient from two buffers in
    turn, as the headline does from three."""
    out = {}

    def entry(workload, n, bytes_per, fn, t0, reps=steps, warm=3):
        t = [t0]

        def run():
            fn(t[0])
            t[0] += 1
        for _ in range(warm):
            run()
        med, mn = _median_ms(torch, run, reps)
        gbps = bytes_per * n / (med * 1e-3) / 1e9
        return {"workload": workload, "shard_len": n, "median_ms": round(med, 4), "min_ms": round(mn, 4),
                "params_per_s": n / (med * 1e-3), "bytes_per_param": bytes_per, "hbm_gbps": round(gbps, 1),
                "frac_of_peak": round(gbps / PEAK_HBM_GBPS, 4)}

    def batch_ms(fn, reps):
        """Average device time per call over `reps` back-to-back calls."""
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

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
        small = n < (1 << 22)
        res = entry(name, n, REDUCE_BYTES_PER_PARAM(n_ranks) + 30, fn, t0, reps=100 if small else steps,
                    warm=20 if small else 3)
        if small:
            # launch-bound: the same calls captured once in a HIP graph and
            # replayed (the step number is fixed in the captured launch);
            # per-call medians from events around each call, and the mean of
            # 100 back-to-back calls with no events in between
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                fn(t0 + 1000)
            for _ in range(20):
                graph.replay()
            med, mn = _median_ms(torch, graph.replay, 100)
            res["graph_replay_median_ms"], res["graph_replay_min_ms"] = round(med, 4), round(mn, 4)
            tt = [t0 + 2000]

            def eager():
                fn(tt[0])
                tt[0] += 1
            res["eager_batch_mean_ms"] = round(batch_ms(eager, 100), 4)
            res["graph_replay_batch_mean_ms"] = round(batch_ms(graph.replay, 100), 4)
            del graph
        del slices, master, m, v, p16, gsum
        torch.cuda.empty_cache()
        return res

    def stats_step(psi, n_ranks, seed, t0, name, student=False, skip_run=False):
        n = zs.partition_layout(psi, n_ranks, 0, 128).shard_len
        master, m, v, p16 = tk.init_shard_state(n, seed, zero_moments=student, device=dev)
        gs = [torch.empty(n, dtype=torch.float16, device=dev) for _ in range(2)]
        for k, g in enumerate(gs):
            if student:
                tk.student_t3_f16_(g, 1e-3 * 65536, seed, tk.STREAM_GRAD + k, redraw_overflow=True)
            else:
                tk.normal_f16_(g, 1e-3 * 65536, seed, tk.STREAM_GRAD + k)
        stats, ws = zs.new_stats(dev), zs.new_workspace(n, dev)

        def fn(t):
            g = gs[t % 2]
            zs.grad_stats(g, stats, inv_grad_scale=INV_SCALE, workspace=ws)
            zs.adam_step(g, master, m, v, p16, step=t, lr=LR, betas=BETAS, eps=EPS, inv_grad_scale=INV_SCALE,
                         stats=stats, stats_precomputed=True)
        res = entry(name, n, UPDATE_BYTES_PER_PARAM + STATS_BYTES_PER_PARAM, fn, t0)
        if skip_run:
            # 0.001% of each gradient set to +inf: the statistics flag the
            # step and every update block leaves before touching the states
            for k, g in enumerate(gs):
                tk.inject_inf_f16_(g, 1e-5, seed + 0xF, tk.STREAM_INF + k)
            ev = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(steps)]
            torch.cuda.synchronize()
            for k in range(steps):
                g = gs[k % 2]
                ev[k][0].record()
                zs.grad_stats(g, stats, inv_grad_scale=INV_SCALE, workspace=ws)
                ev[k][1].record()
                zs.adam_step(g, master, m, v, p16, step=t0 + 500, lr=LR, betas=BETAS, eps=EPS,
                             inv_grad_scale=INV_SCALE, stats=stats, stats_precomputed=True)
                ev[k][2].record()
            torch.cuda.synchronize()
            flag = zs.read_stats(stats)[0]

            def med(xs):
                xs = sorted(xs)
                return (xs[(len(xs) - 1) // 2] + xs[len(xs) // 2]) / 2
            whole = med([a.elapsed_time(c) for a, _, c in ev])
            res["skipped_step"] = {
                "overflow_flag": flag, "median_ms": round(whole, 4),
                "statistics_median_ms": round(med([a.elapsed_time(b) for a, b, _ in ev]), 4),
                "update_exit_median_ms": round(med([b.elapsed_time(c) for _, b, c in ev]), 4),
                "statistics_gbps": round(STATS_BYTES_PER_PARAM * n / (med([a.elapsed_time(b) for a, b, _ in ev])
                                                                      * 1e-3) / 1e9, 1)}
        del master, m, v, p16, gs
        torch.cuda.empty_cache()
        return res

    out["tiny_n4"] = reduce_step(1_048_576, 4, 0xC1, 1e-3 * 65536, 2.0 ** -18, 1,
                                 "tiny: psi=1,048,576, N=4, reduce of 4 slices + update (fp32 sum); "
                                 "launch-bound and cache-resident, not a roofline figure")
    out["7p5b_n64"] = reduce_step(7_500_000_000, 64, 0xC3, 1e-3 * 4096, 2.0 ** -18, 10,
                                  "7.5B at N=64: reduce of 64 slices + update (fp32 sum)")
    out["7b_n8"] = stats_step(7_000_000_000, 8, 0xC4, 1000, "7B at N=8: statistics + update (fp16 grad); "
                              "skipped_step: the same with 0.001% of the gradient +inf", skip_run=True)
    out["1p5b_n1"] = stats_step(1_500_000_000, 1, 0xC5, 1,
                                "GPT-2-XL unpartitioned (N=1): statistics + update (fp16 Student-t(3) grad, "
                                "overflowing draws redrawn)", student=True)
    return out


class _one_core:
    """Pins this process to one host core while the (single-threaded) oracle
    runs, and restores the affinity afterwards."""

    def __enter__(self):
        self.allowed = os.sched_getaffinity(0) if hasattr(os, "sched_getaffinity") else None
        self.core = None
        if self.allowed:
            self.core = min(self.allowed)
            os.sched_setaffinity(0, {self.core})
        return self

    def __exit__(self, *exc):
        if self.allowed:
            os.sched_setaffinity(0, self.allowed)


def _repeat(fn, target_s):
    """Calls fn() until target_s seconds have passed; (calls, seconds)."""
    reps, t0 = 0, time.perf_counter()
    while True:
        fn(reps)
        reps += 1
        el = time.perf_counter() - t0
        if el >= target_s:
            return reps, el


def _host_u16(torch, t):
    import numpy as np
    return t.cpu().view(torch.int16).numpy().view(np.uint16).copy()


def _host_state(torch, master, m, v, p16):
    return [master.cpu().numpy().copy(), m.cpu().numpy().copy(), v.cpu().numpy().copy(), _host_u16(torch, p16)]


def cpu_baseline(torch, zs, tk, dev, g, master, m, v, p16, gpu_rates, target_s=6.0):
    """The oracle (single-threaded C, untuned) on one pinned host core, on
    bounded samples of the workloads, each timed for about target_s seconds
    (the 1.5e9 flag scan once, whole):
      gpt2xl_n4  the first 2^24 parameters of the 375,000,064 shard:
                 statistics + update (the headline);
      7p5b_n64   the first 2^22 rows of all 64 slices of the 117,187,584
                 shard: the reduce alone (132 B/param), and reduce +
                 statistics + update on the sum;
      7b_n8      the first 2^24 parameters of the 875,000,064 shard:
                 statistics + update;
      1p5b_n1    one step's check of the unpartitioned run: the update of
                 1,048,576 sampled parameters plus the statistics (flag and
                 sum of squares) over the whole 1.5e9-value gradient.
    gpu_rates: the GPU's params/s for the same workloads in this run (None
    where not measured), for the ratios."""
    import numpy as np

    import oracle
    out = {}
    ratio = lambda a, b: round(a / b, 1) if a and b else None  # noqa: E731

    # ---- inputs, prepared on the GPU with the workloads' generators (the
    # counter-based generator gives the leading elements of each tensor)
    n2 = 1 << 24
    c2 = [_host_u16(torch, g[:n2]), *_host_state(torch, master[:n2], m[:n2], v[:n2], p16[:n2])]
    n3 = 1 << 22
    sl3 = [_host_u16(torch, tk.normal_f16_(torch.empty(n3, dtype=torch.float16, device=dev), 1e-3 * 4096, 0xC3,
                                           tk.STREAM_GRAD + r)) for r in range(64)]
    st3 = _host_state(torch, *tk.init_shard_state(n3, 0xC3, zero_moments=False, device=dev))
    n4 = 1 << 24
    g4 = _host_u16(torch, tk.normal_f16_(torch.empty(n4, dtype=torch.float16, device=dev), 1e-3 * 65536, 0xC4,
                                         tk.STREAM_GRAD))
    st4 = _host_state(torch, *tk.init_shard_state(n4, 0xC4, zero_moments=False, device=dev))
    n5 = 1_500_000_000
    g5d = tk.student_t3_f16_(torch.empty(n5, dtype=torch.float16, device=dev), 1e-3 * 65536, 0xC5, tk.STREAM_GRAD,
                             redraw_overflow=True)
    rng = np.random.default_rng(0xC5)
    stride = n5 // 1_048_576
    idx = np.arange(1_048_576, dtype=np.int64) * stride + rng.integers(0, stride, 1_048_576)
    idx_d = torch.from_numpy(idx).to(dev)
    m5 = tk.normal_f32_(torch.empty(n5, dtype=torch.float32, device=dev), 0.0, 0.02, 0xC5, tk.STREAM_MASTER)
    st5 = [m5.index_select(0, idx_d).cpu().numpy().copy(), np.zeros(idx.size, np.float32),
           np.zeros(idx.size, np.float32), np.zeros(idx.size, np.uint16)]
    del m5
    g5 = _host_u16(torch, g5d)
    del g5d, idx_d
    torch.cuda.empty_cache()
    g5s = g5[idx].copy()
    kw = dict(lr=LR, beta1=BETAS[0], beta2=BETAS[1], eps=EPS)

    def step_fn(gh, st, t0, s):
        def f(k):
            rc, _, _ = oracle.shard_adam_step(gh, *st, step=t0 + k, inv_scale=s, **kw)
            assert rc == 0
        return f

    with _one_core() as pin:
        reps, el = _repeat(step_fn(c2[0], c2[1:], T0, INV_SCALE), target_s)
        r2 = n2 * reps / el
        out["gpt2xl_n4"] = {"params_per_s": r2, "gbps": round(r2 * 30 / 1e9, 3),
                            "gpu_over_oracle": ratio(gpu_rates.get("gpt2xl_n4"), r2),
                            "sample": f"first {n2:,} params of the 375,000,064-param shard, statistics + update, "
                                      f"{reps} repetitions in {el:.1f} s"}

        def red(k):
            oracle.grad_reduce(sl3)
        reps, el = _repeat(red, target_s / 2)
        rr = n3 * reps / el

        def red_step(k):
            gs = oracle.grad_reduce(sl3)
            rc, _, _ = oracle.shard_adam_step(gs, *st3, step=10 + k, inv_scale=2.0 ** -18, **kw)
            assert rc == 0
        reps2, el2 = _repeat(red_step, target_s / 2)
        rs = n3 * reps2 / el2
        out["7p5b_n64"] = {"reduce_params_per_s": rr, "reduce_gbps": round(rr * REDUCE_BYTES_PER_PARAM(64) / 1e9, 3),
                           "reduce_gpu_over_oracle": ratio(gpu_rates.get("7p5b_n64_reduce"), rr),
                           "step_params_per_s": rs, "step_gbps": round(rs * (REDUCE_BYTES_PER_PARAM(64) + 30) / 1e9, 3),
                           "step_gpu_over_oracle": ratio(gpu_rates.get("7p5b_n64_step"), rs),
                           "sample": f"first {n3:,} rows of all 64 slices of the 117,187,584-param shard: reduce "
                                     f"({reps} in {el:.1f} s), reduce + statistics + update on the fp32 sum "
                                     f"({reps2} in {el2:.1f} s)"}
        reps, el = _repeat(step_fn(g4, st4, T0, INV_SCALE), target_s)
        r4 = n4 * reps / el
        out["7b_n8"] = {"params_per_s": r4, "gbps": round(r4 * 30 / 1e9, 3),
                        "gpu_over_oracle": ratio(gpu_rates.get("7b_n8"), r4),
                        "sample": f"first {n4:,} params of the 875,000,064-param shard, statistics + update, "
                                  f"{reps} repetitions in {el:.1f} s"}

        def upd5(k):
            assert oracle.adam_apply(g5s, *st5, step=1 + k, inv_scale=INV_SCALE, overflow=0, **kw) == 0
        reps, el = _repeat(upd5, 1.0)
        ru = idx.size * reps / el
        t_scan = time.perf_counter()
        flag, _ = oracle.grad_stats(g5, INV_SCALE)
        t_scan = time.perf_counter() - t_scan
        assert flag == 0
        rscan = n5 / t_scan
        per_step = idx.size / ru + t_scan
        # the oracle's rate for a whole step of the 1.5e9 model (update of all
        # parameters at the subset's rate, plus the full statistics)
        r5 = 1.0 / (1.0 / ru + 1.0 / rscan)
        out["1p5b_n1"] = {"subset_update_params_per_s": ru, "flag_scan_params_per_s": rscan,
                          "flag_scan_gbps": round(rscan * 2 / 1e9, 3), "flag_scan_s": round(t_scan, 2),
                          "per_step_check_s": round(per_step, 2), "whole_step_params_per_s": r5,
                          "gpu_over_oracle": ratio(gpu_rates.get("1p5b_n1"), r5),
                          "sample": f"update of {idx.size:,} stratified sampled params ({reps} in {el:.1f} s) + "
                                    f"statistics over the whole {n5:,}-value gradient (once)"}
        core = pin.core
    cpu_model = platform.processor() or "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    head = out["gpt2xl_n4"]
    return {"value": head["params_per_s"], "unit": "params/s", "cores": 1, "kind": "oracle",
            "sample": head["sample"], "gbps": head["gbps"], "gpu_over_oracle": head["gpu_over_oracle"],
            "pinned_core": core, "host_cpu": cpu_model, "host_threads": os.cpu_count(),
            "nproc": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count(),
            "configs": out}


def host_adam_secondary(torch, g, master, m, v, p16, steps=5, warm=8):
    """The multi-core SIMD host step (ZeRO-Offload's CPU Adam) on the whole
    shard in host memory: statistics + update, all OpenMP threads, after
    `warm` untimed steps (a fresh allocation's first passes over host memory
    run well below the steady rate).  Beside it, the same host's attainable
    rate: an in-place multi-threaded read-modify-write (x += 0, 8 B/element)
    over the master array with torch's CPU kernels."""
    import numpy as np

    from zero_partitioned_mixed_flat_amd import host_adam as ha
    n = master.numel()
    g_h = g.cpu().view(torch.int16).numpy().view(np.uint16).copy()
    st = [master.cpu().numpy().copy(), m.cpu().numpy().copy(), v.cpu().numpy().copy(),
          p16.cpu().view(torch.int16).numpy().view(np.uint16).copy()]
    threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or (os.cpu_count() or 1)
    isa = ha.set_isa(0)
    for k in range(warm):
        ha.adam_step(g_h, *st, step=T0 + k, lr=LR, betas=BETAS, eps=EPS, inv_grad_scale=INV_SCALE, threads=threads)
    t0 = time.perf_counter()
    for k in range(steps):
        ha.adam_step(g_h, *st, step=T0 + warm + k, lr=LR, betas=BETAS, eps=EPS, inv_grad_scale=INV_SCALE,
                     threads=threads)
    el = (time.perf_counter() - t0) / steps
    gbps = (UPDATE_BYTES_PER_PARAM + STATS_BYTES_PER_PARAM) * n / el / 1e9
    x = torch.from_numpy(st[0])
    for _ in range(3):
        x.add_(0.0)
    t0 = time.perf_counter()
    for _ in range(steps):
        x.add_(0.0)
    rmw = 8 * n / ((time.perf_counter() - t0) / steps) / 1e9
    return {"value": n / el, "unit": "params/s", "cores": threads, "kind": "host SIMD+OpenMP step",
            "isa": ha.ISA_NAMES[isa], "ms_per_step": round(el * 1e3, 2), "host_gbps": round(gbps, 1),
            "host_rmw_ceiling_gbps": round(rmw, 1), "rmw_threads": torch.get_num_threads(),
            "frac_of_host_rmw_ceiling": round(gbps / rmw, 4),
            "sample": f"the whole {n:,}-param shard in host memory, statistics + update, {warm} untimed and "
                      f"{steps} timed steps"}


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
    # three gradients of the workload's recipe (seeded streams), used in turn
    grads = [tk.normal_f16_(torch.empty(L, dtype=torch.float16, device=dev), 1e-3 * 65536, SEED,
                            tk.STREAM_GRAD + k) for k in range(N_GRAD_BUFFERS)]
    g = grads[0]
    stats = zs.new_stats(dev)
    ws = zs.new_workspace(L, dev)
    torch.cuda.synchronize()

    ceil = ceiling(torch, tk, dev)
    log(f"ceiling: {ceil}")

    def one_step(t, grad, ev=None):
        layout = zs.partition_layout(PSI, N_RANKS, RANK, ALIGN)          # a1 (host)
        assert layout.shard_len == L
        zs.grad_stats(grad, stats, inv_grad_scale=INV_SCALE, workspace=ws)  # a3 (2 kernels)
        if ev is not None:
            ev[0].record()
        zs.adam_step(grad, master, m, v, p16, step=t, lr=LR, betas=BETAS, eps=EPS, inv_grad_scale=INV_SCALE,
                     stats=stats, stats_precomputed=True)                # a4-a8 (1 kernel)
        if ev is not None:
            ev[1].record()

    def timed_loop(t0, buffers):
        """K steps, step k on buffers[k % len(buffers)]: wall time, the
        update launches timed by events around them on the stream, and the
        statistics (+ finalize and the kernel boundaries) as the time from one
        step's update end to the next step's update start.  Each event record
        adds about 2.5 us of stream time, so a step carries only the two
        around its update."""
        evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(2)) for _ in range(args.steps)]
        torch.cuda.synchronize()
        t_start = time.perf_counter()
        for k in range(args.steps):
            one_step(t0 + k, buffers[k % len(buffers)], evs[k])
        torch.cuda.synchronize()
        wall = time.perf_counter() - t_start
        upd = [e[0].elapsed_time(e[1]) for e in evs]
        sta = [evs[k - 1][1].elapsed_time(evs[k][0]) for k in range(1, len(evs))]
        return wall, upd, sta

    for i in range(args.warmup):
        one_step(T0 + i, grads[i % N_GRAD_BUFFERS])
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} steps done; flag/sumsq = {zs.read_stats(stats)}")

    wall, upd_ms, stats_ms = timed_loop(T0 + args.warmup, grads)
    stats_avg_s = sum(stats_ms) / len(stats_ms) * 1e-3 if stats_ms else None
    upd_avg_s = sum(upd_ms) / len(upd_ms) * 1e-3
    upd_sorted = sorted(upd_ms)
    upd_median_ms = (upd_sorted[(len(upd_ms) - 1) // 2] + upd_sorted[len(upd_ms) // 2]) / 2
    overflow, sumsq = zs.read_stats(stats)
    log(f"timed {args.steps} steps over {N_GRAD_BUFFERS} gradient buffers: wall {wall * 1e3:.3f} ms, "
        f"update avg {upd_avg_s * 1e3:.4f} ms, overflow={overflow}")
    # the same loop with one gradient reused by every step, for comparison
    wall1, upd1, stats1 = timed_loop(T0 + args.warmup + args.steps, [g])
    single_buffer = {"ms_per_step": round(wall1 / args.steps * 1e3, 4), "value": L / (wall1 / args.steps),
                     "update_avg_ms": round(sum(upd1) / len(upd1), 4),
                     "statistics_avg_ms": round(sum(stats1) / len(stats1), 4) if stats1 else None}
    log(f"single gradient buffer: {single_buffer}")

    step_s = wall / args.steps
    value = L / step_s
    whole_gbps = (UPDATE_BYTES_PER_PARAM + STATS_BYTES_PER_PARAM) * L / step_s / 1e9
    upd_gbps = UPDATE_BYTES_PER_PARAM * L / upd_avg_s / 1e9
    traffic = counter_traffic()
    stats_traffic = counter_traffic(STATS_COUNTERS_FILE)
    # HBM bytes of the whole step from the committed counter summaries
    # (statistics + update; the 16-byte finalize is negligible), over the
    # wall time of a step in this run
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
            gk = grads[k % N_GRAD_BUFFERS]
            zs.grad_stats(gk, stats, inv_grad_scale=INV_SCALE, workspace=ws)
            a.record()
            zs.adam_step(gk, master, m, v, p16, step=T0 + 100 + k, lr=LR, betas=BETAS, eps=EPS,
                         inv_grad_scale=INV_SCALE, max_grad_norm=1.0, stats=stats, stats_precomputed=True)
            b.record()
            clip_ms.append((a, b))
        torch.cuda.synchronize()
        clip_avg = sum(a.elapsed_time(b) for a, b in clip_ms) / len(clip_ms)
        qwz = qwz_secondary(torch, zs, tk, dev, args.steps, grads, master, m, v, p16, stats, ws, T0 + 200)
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
        oc = (secondary or {}).get("other_configs", {})
        gpu_rates = {"gpt2xl_n4": value,
                     "7p5b_n64_reduce": (secondary or {}).get("reduce_n64", {}).get("params_per_s"),
                     "7p5b_n64_step": oc.get("7p5b_n64", {}).get("params_per_s"),
                     "7b_n8": oc.get("7b_n8", {}).get("params_per_s"),
                     "1p5b_n1": oc.get("1p5b_n1", {}).get("params_per_s")}
        cpu = cpu_baseline(torch, zs, tk, dev, g, master, m, v, p16, gpu_rates)
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
        "gradient_buffers": N_GRAD_BUFFERS, "single_buffer": single_buffer,
        # not measured in this run: the committed counter summaries' bytes
        # (valid only for the kernel sources they were taken with) over this
        # run's step time
        "hbm_gbps_from_committed_counters": (
            {"value": round(step_counter_bytes / step_s / 1e9, 1),
             "files": [os.path.relpath(COUNTERS_FILE, ROOT), os.path.relpath(STATS_COUNTERS_FILE, ROOT)],
             "kernel_source_sha256": kernel_source_hash()} if step_counter_bytes else None),
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
        "statistics": ({"kernels": "grad_stats_kernel<f16> + finalize_stats_kernel, with the kernel boundaries "
                                   "between one update's end and the next update's start", "bound": "hbm",
                        "avg_ms": round(stats_avg_s * 1e3, 4),
                        "achieved": round(STATS_BYTES_PER_PARAM * L / stats_avg_s / 1e9, 1), "unit": "GB/s",
                        "frac": round(STATS_BYTES_PER_PARAM * L / stats_avg_s / 1e9 / PEAK_HBM_GBPS, 4),
                        "traffic": stats_traffic, "algorithmic_bytes_per_launch": STATS_BYTES_PER_PARAM * L}
                       if stats_avg_s else None),
        "ceiling": ceil,
        "secondary": secondary,
        "cpu_baseline": cpu,
        "host_adam": host,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
