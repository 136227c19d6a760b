"""ctypes binding of libzero_testkit.so (csrc/zero_testkit.h): seeded
synthetic inputs on the device and plain streaming reference kernels.  Used
by the tests and the benchmark; holds none of the optimizer step's
arithmetic and loads none of the optimizer library's code (the probes of
that code are in probes.py).

Input recipe of the workloads (sigma is a standard deviation):
  master  ~ N(0, 0.02)           fp32
  m       ~ N(0, 1e-4) or 0      fp32
  v       ~ |N(0, 1e-6)| or 0    fp32
  grad    f16(N(0, 1e-3) * loss_scale), or f16(1e-3 * t3 * loss_scale)
Each tensor has its own Philox stream id; per-step gradients use stream
``stream + step``.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

LIB_PATH = _build.library_path("libzero_testkit.so")
if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it (python zero_partitioned_mixed_flat_amd/build.py)")

# PyTorch ships its own HIP runtime (SONAME libamdhip64.so.7).  Loading torch
# first makes this library bind to that same runtime; loading it first would
# bring a second HIP runtime into the process, which then finds no device.
import torch  # noqa: E402,F401

_lib = ctypes.CDLL(LIB_PATH)
_p, _i32, _i64, _u32, _u64, _dbl = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32,
                                    ctypes.c_uint64, ctypes.c_double)
_lib.zero_testkit_philox.argtypes = [_p, _i64, _u64, _u32, _p]
_lib.zero_testkit_normal_f32.argtypes = [_p, _i64, _dbl, _dbl, _i32, _u64, _u32, _p]
_lib.zero_testkit_normal_f16.argtypes = [_p, _i64, _dbl, _u64, _u32, _p]
_lib.zero_testkit_student_t3_f16.argtypes = [_p, _i64, _dbl, _i32, _u64, _u32, _p]
_lib.zero_testkit_inject_inf_f16.argtypes = [_p, _i64, _dbl, _u64, _u32, _p]
_lib.zero_testkit_copy_f32.argtypes = [_p, _p, _i64, _p]
_lib.zero_testkit_read_f32.argtypes = [_p, _i64, _p, _i32, _p]
_lib.zero_testkit_read_slices.argtypes = [_p, _i32, _i64, _p, _p, _i32, _p]
_lib.zero_testkit_last_error.argtypes = []
_lib.zero_testkit_last_error.restype = ctypes.c_char_p
for _f in ("zero_testkit_philox", "zero_testkit_normal_f32", "zero_testkit_normal_f16",
           "zero_testkit_student_t3_f16", "zero_testkit_inject_inf_f16", "zero_testkit_copy_f32",
           "zero_testkit_read_f32", "zero_testkit_read_slices"):
    getattr(_lib, _f).restype = ctypes.c_int

# Philox stream ids of the workload tensors
STREAM_MASTER, STREAM_M, STREAM_V, STREAM_GRAD, STREAM_INF = 1, 2, 3, 16, 9


def library() -> ctypes.CDLL:
    return _lib


def _stream():
    import torch
    return int(torch.cuda.current_stream().cuda_stream)


def _ok(rc: int, what: str):
    if rc != 0:
        detail = _lib.zero_testkit_last_error().decode() if rc == -4 else "bad argument"
        raise RuntimeError(f"{what} failed with {rc}: {detail}")


def philox(n_blocks: int, seed: int, stream: int, device="cuda"):
    import torch
    out = torch.empty(4 * n_blocks, dtype=torch.int32, device=device)
    _ok(_lib.zero_testkit_philox(out.data_ptr(), n_blocks, seed, stream, _stream()), "philox")
    return out


def normal_f32_(t, mean: float, std: float, seed: int, stream: int, abs_value=False):
    import torch
    assert t.dtype == torch.float32 and t.is_contiguous()
    _ok(_lib.zero_testkit_normal_f32(t.data_ptr(), t.numel(), mean, std, int(abs_value), seed, stream,
                                     _stream()), "normal_f32")
    return t


def normal_f16_(t, scale: float, seed: int, stream: int):
    import torch
    assert t.dtype == torch.float16 and t.is_contiguous()
    _ok(_lib.zero_testkit_normal_f16(t.data_ptr(), t.numel(), scale, seed, stream, _stream()), "normal_f16")
    return t


def student_t3_f16_(t, scale: float, seed: int, stream: int, redraw_overflow=False):
    import torch
    assert t.dtype == torch.float16 and t.is_contiguous()
    _ok(_lib.zero_testkit_student_t3_f16(t.data_ptr(), t.numel(), scale, int(redraw_overflow), seed, stream,
                                         _stream()), "student_t3_f16")
    return t


def inject_inf_f16_(t, prob: float, seed: int, stream: int = STREAM_INF):
    import torch
    assert t.dtype == torch.float16 and t.is_contiguous()
    _ok(_lib.zero_testkit_inject_inf_f16(t.data_ptr(), t.numel(), prob, seed, stream, _stream()), "inject_inf")
    return t


def copy_f32(src, dst):
    _ok(_lib.zero_testkit_copy_f32(src.data_ptr(), dst.data_ptr(), src.numel(), _stream()), "copy_f32")


def read_f32(src, sink):
    _ok(_lib.zero_testkit_read_f32(src.data_ptr(), src.numel(), sink.data_ptr(), sink.numel(), _stream()),
        "read_f32")


def read_slices(slices, sink, out=None):
    """Streaming reference over many fp16 slices (zero_testkit_read_slices):
    reads them all; with `out` (int32, same length) also writes the XOR of
    the slices' values per element."""
    import ctypes as _c
    n = len(slices)
    length = slices[0].numel()
    ptrs = (_c.c_void_p * n)(*[t.data_ptr() for t in slices])
    _ok(_lib.zero_testkit_read_slices(_c.cast(ptrs, _c.c_void_p), n, length,
                                      out.data_ptr() if out is not None else None, sink.data_ptr(), sink.numel(),
                                      _stream()), "read_slices")


def init_shard_state(length: int, seed: int, *, zero_moments: bool, device="cuda"):
    """master ~ N(0,0.02); m ~ N(0,1e-4), v ~ |N(0,1e-6)| (or zeros); p16 = 0."""
    import torch
    master = normal_f32_(torch.empty(length, dtype=torch.float32, device=device), 0.0, 0.02, seed, STREAM_MASTER)
    if zero_moments:
        m = torch.zeros(length, dtype=torch.float32, device=device)
        v = torch.zeros(length, dtype=torch.float32, device=device)
    else:
        m = normal_f32_(torch.empty(length, dtype=torch.float32, device=device), 0.0, 1e-4, seed, STREAM_M)
        v = normal_f32_(torch.empty(length, dtype=torch.float32, device=device), 0.0, 1e-6, seed, STREAM_V,
                        abs_value=True)
    p16 = torch.zeros(length, dtype=torch.float16, device=device)
    return master, m, v, p16


# ------------------------------------------------------- host Philox (numpy)
_M0, _M1 = np.uint64(0xD2511F53), np.uint64(0xCD9E8D57)
_W0, _W1 = np.uint32(0x9E3779B9), np.uint32(0xBB67AE85)


def philox_host(counters: np.ndarray, key: tuple[int, int]) -> np.ndarray:
    """Philox4x32-10 of an [n, 4] uint32 counter array on the host (numpy),
    the same definition as the device generator."""
    c = counters.astype(np.uint32).copy()
    k0 = np.uint32(key[0])
    k1 = np.uint32(key[1])
    mask = np.uint64(0xFFFFFFFF)
    for r in range(10):
        if r > 0:
            k0 = np.uint32((int(k0) + int(_W0)) & 0xFFFFFFFF)
            k1 = np.uint32((int(k1) + int(_W1)) & 0xFFFFFFFF)
        p0 = c[:, 0].astype(np.uint64) * _M0
        p1 = c[:, 2].astype(np.uint64) * _M1
        hi0, lo0 = (p0 >> np.uint64(32)).astype(np.uint32), (p0 & mask).astype(np.uint32)
        hi1, lo1 = (p1 >> np.uint64(32)).astype(np.uint32), (p1 & mask).astype(np.uint32)
        c = np.stack([hi1 ^ c[:, 1] ^ k0, lo1, hi0 ^ c[:, 3] ^ k1, lo0], axis=1)
    return c
