"""ctypes binding of libzero_probes.so (csrc/zero_probes.h): device probes
of the optimizer library's own code -- its arithmetic helpers and its
streaming-store policy -- for the tests and the benchmark."""
from __future__ import annotations

import ctypes
import os

from . import build as _build

LIB_PATH = _build.library_path("libzero_probes.so")
if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it (python zero_partitioned_mixed_flat_amd/build.py)")

# Loading torch first binds this library to torch's HIP runtime (as for the
# other libraries of the package).
import torch  # noqa: E402,F401

_lib = ctypes.CDLL(LIB_PATH)
_p, _i64, _dbl = ctypes.c_void_p, ctypes.c_int64, ctypes.c_double
_lib.zero_probes_arith_f32.argtypes = [_p, _p, _p, _i64, _p, _p, _p, _p, _p]
_lib.zero_probes_bias_correction.argtypes = [_dbl, _p, _i64, _p, _p]
_lib.zero_probes_rmw_f32.argtypes = [_p, _i64, _p]
_lib.zero_probes_last_error.argtypes = []
_lib.zero_probes_last_error.restype = ctypes.c_char_p
for _f in ("zero_probes_arith_f32", "zero_probes_bias_correction", "zero_probes_rmw_f32"):
    getattr(_lib, _f).restype = ctypes.c_int


def library() -> ctypes.CDLL:
    return _lib


def _stream():
    import torch
    return int(torch.cuda.current_stream().cuda_stream)


def _ok(rc: int, what: str):
    if rc != 0:
        detail = _lib.zero_probes_last_error().decode() if rc == -4 else "bad argument"
        raise RuntimeError(f"{what} failed with {rc}: {detail}")


def rmw_f32(p):
    """p += 1 in place with the library's streaming-store policy."""
    _ok(_lib.zero_probes_rmw_f32(p.data_ptr(), p.numel(), _stream()), "rmw_f32")


def bias_correction(beta: float, t):
    """The library's device-side (float)(1 - beta^t) for an int64 device tensor t."""
    import torch
    assert t.dtype == torch.int64 and t.is_contiguous()
    out = torch.empty(t.numel(), dtype=torch.float32, device=t.device)
    _ok(_lib.zero_probes_bias_correction(float(beta), t.data_ptr(), t.numel(), out.data_ptr(), _stream()),
        "bias_correction")
    return out


def arith_f32(a, b, h):
    """(a / b, sqrt(a), f16(a) bits, f32(h)) on the device with the library's
    primitives; a, b float32 and h int16 (fp16 bits) device tensors of one length."""
    import torch
    n = a.numel()
    assert b.numel() == n and h.numel() == n and a.dtype == b.dtype == torch.float32 and h.dtype == torch.int16
    quot, root, wide = (torch.empty_like(a) for _ in range(3))
    half = torch.empty(n, dtype=torch.int16, device=a.device)
    _ok(_lib.zero_probes_arith_f32(a.data_ptr(), b.data_ptr(), h.data_ptr(), n, quot.data_ptr(), root.data_ptr(),
                                   half.data_ptr(), wide.data_ptr(), _stream()), "arith_f32")
    return quot, root, half, wide
