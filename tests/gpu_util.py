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
