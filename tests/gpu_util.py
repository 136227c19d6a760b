"""Shared helpers of the GPU parity tests: device/host copies and the parity
bar (overflow flag and layout bit-exact; fp32 max relative error 1e-6; fp16
within 1 ulp; the sum of squares within 1e-10 relative)."""
import sys

import numpy as np

FP32_REL = 1e-6
F16_ULP = 1
SUMSQ_REL = 1e-10


def say(*args):
    print(*args, flush=True)
    sys.stdout.flush()


def require_gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return torch.device("cuda:0")


def host_f32(t) -> np.ndarray:
    return t.detach().cpu().numpy().astype(np.float32, copy=False)


def host_u16(t) -> np.ndarray:
    return t.detach().cpu().view(__import__("torch").int16).numpy().view(np.uint16)


def _ordered_f16(bits: np.ndarray) -> np.ndarray:
    b = bits.astype(np.int32)
    return np.where(b & 0x8000, -(b & 0x7FFF), b & 0x7FFF)


def assert_f32_close(got: np.ndarray, ref: np.ndarray, name: str) -> int:
    """Max relative error <= 1e-6 (exact where the reference is 0 or not
    finite).  Returns the number of elements that are not bit-identical."""
    g64, r64 = got.astype(np.float64), ref.astype(np.float64)
    both_nan = np.isnan(g64) & np.isnan(r64)
    same = (got.view(np.uint32) == ref.view(np.uint32)) | both_nan
    err = np.abs(g64 - r64)
    ok = same | (np.isfinite(r64) & (err <= FP32_REL * np.abs(r64)))
    if not ok.all():
        i = int(np.argmin(ok))
        raise AssertionError(f"{name}: {int((~ok).sum())} elements beyond rel {FP32_REL}; "
                             f"first at {i}: got {got[i]!r} want {ref[i]!r}")
    return int((~same).sum())


def assert_f16_close(got: np.ndarray, ref: np.ndarray, name: str) -> int:
    same = got == ref
    nan_g = ((got & 0x7C00) == 0x7C00) & ((got & 0x3FF) != 0)
    nan_r = ((ref & 0x7C00) == 0x7C00) & ((ref & 0x3FF) != 0)
    close = np.abs(_ordered_f16(got) - _ordered_f16(ref)) <= F16_ULP
    ok = same | (nan_g & nan_r) | (close & ~nan_g & ~nan_r)
    if not ok.all():
        i = int(np.argmin(ok))
        raise AssertionError(f"{name}: {int((~ok).sum())} fp16 elements beyond 1 ulp; first at {i}: "
                             f"got {got[i]:#06x} want {ref[i]:#06x}")
    return int((~same).sum())


def assert_stats(gpu, ref, name: str):
    (gf, gs), (rf, rs) = gpu, ref
    assert gf == rf, f"{name}: overflow flag {gf} != oracle {rf}"
    if rf == 0:
        assert abs(gs - rs) <= SUMSQ_REL * abs(rs) + 1e-300, f"{name}: sumsq {gs!r} vs oracle {rs!r}"


def assert_state_parity(gpu, ref, name: str):
    """gpu, ref = (master, m, v, p16) host arrays.  Returns inexact counts."""
    counts = {}
    for k, (a, b) in zip(("master", "m", "v"), zip(gpu[:3], ref[:3])):
        counts[k] = assert_f32_close(a, b, f"{name}.{k}")
    counts["p16"] = assert_f16_close(gpu[3], ref[3], f"{name}.p16")
    return counts


# ------------------------------------------------ oracle over large arrays
# The oracle is single-threaded; at full workload sizes the tests run it on
# independent contiguous chunks in a thread pool (ctypes releases the GIL).
# Chunking is exact for the elementwise update and reduce (separability,
# pinned bit-exact on the CPU); the statistics combine per-chunk flags by OR
# and per-chunk compensated sums with math.fsum.
import concurrent.futures as _cf
import math as _math
import os as _os

THREADS = max(1, min(16, _os.cpu_count() or 1))


def _chunks(n, parts):
    step = -(-n // parts) if n else 1
    step = ((step + 1023) // 1024) * 1024
    return [(a, min(n, a + step)) for a in range(0, n, step)]


def oracle_stats_full(g_host, s):
    import oracle
    with _cf.ThreadPoolExecutor(THREADS) as ex:
        res = list(ex.map(lambda ab: oracle.grad_stats(g_host[ab[0]:ab[1]], s), _chunks(g_host.size, 4 * THREADS)))
    flag = 1 if any(f for f, _ in res) else 0
    return flag, _math.fsum(x for _, x in res)


def oracle_apply_full(g_host, master, m, v, p16, *, step, lr, betas, eps, s, overflow):
    import oracle

    def run(ab):
        a, b = ab
        sl = slice(a, b)
        return oracle.adam_apply(g_host[sl], master[sl], m[sl], v[sl], p16[sl], step=step, lr=lr,
                                 beta1=betas[0], beta2=betas[1], eps=eps, inv_scale=s, overflow=overflow)
    with _cf.ThreadPoolExecutor(THREADS) as ex:
        assert all(rc == 0 for rc in ex.map(run, _chunks(master.size, 4 * THREADS)))


def oracle_reduce_full(slices_host):
    import numpy as np

    import oracle
    n = slices_host[0].size
    out = np.empty(n, dtype=np.float32)

    def run(ab):
        a, b = ab
        out[a:b] = oracle.grad_reduce([sl[a:b] for sl in slices_host])
    with _cf.ThreadPoolExecutor(THREADS) as ex:
        list(ex.map(run, _chunks(n, 4 * THREADS)))
    return out


def stratified_sample(n, count, seed, edge=4096):
    """One seeded index per stratum of n // count elements, plus the first
    and last `edge` indices (the ragged tail), sorted and unique."""
    import numpy as np
    rng = np.random.default_rng(seed)
    stride = n // count
    idx = np.arange(count, dtype=np.int64) * stride + rng.integers(0, stride, count)
    idx = np.concatenate([np.arange(min(edge, n)), idx, np.arange(max(0, n - edge), n)])
    return np.unique(idx[idx < n])


def oracle_qwz_quantize_full(x16):
    """The oracle's qwZ encoding of a large fp16 array, on chunks whose
    boundaries are multiples of 1024 (so every block lies in one chunk)."""
    import numpy as np

    import oracle
    n = x16.size
    codes = np.empty(n, dtype=np.int8)
    scales = np.empty(-(-n // oracle.QWZ_BLOCK), dtype=np.float32)

    def run(ab):
        a, b = ab
        c, s = oracle.qwz_quantize(x16[a:b])
        codes[a:b] = c
        scales[a // oracle.QWZ_BLOCK:a // oracle.QWZ_BLOCK + s.size] = s
    with _cf.ThreadPoolExecutor(THREADS) as ex:
        list(ex.map(run, _chunks(n, 4 * THREADS)))
    return codes, scales


def oracle_qwz_dequantize_full(codes, scales):
    import numpy as np

    import oracle
    n = codes.size
    out = np.empty(n, dtype=np.uint16)

    def run(ab):
        a, b = ab
        blk = a // oracle.QWZ_BLOCK
        out[a:b] = oracle.qwz_dequantize(codes[a:b], scales[blk:blk + -(-(b - a) // oracle.QWZ_BLOCK)])
    with _cf.ThreadPoolExecutor(THREADS) as ex:
        list(ex.map(run, _chunks(n, 4 * THREADS)))
    return out
