"""ctypes binding of libzero_host_adam.so (include/zero_host_adam.h): the
shard Adam step on the host cores, SIMD + OpenMP, with the same arithmetic as
the GPU library.  Argument marshalling only; numpy arrays in host memory."""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

LIB_PATH = _build.library_path("libzero_host_adam.so")
if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build the libraries first "
                      "(python zero_partitioned_mixed_flat_amd/build.py)")

_lib = ctypes.CDLL(LIB_PATH)

F16, F32 = 1, 2
ISA_SCALAR, ISA_AVX2, ISA_AVX512 = 1, 2, 3
ISA_NAMES = {ISA_SCALAR: "scalar+f16c", ISA_AVX2: "avx2+f16c", ISA_AVX512: "avx512"}


class _HParams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_double), ("beta1", ctypes.c_double), ("beta2", ctypes.c_double),
                ("eps", ctypes.c_double), ("max_grad_norm", ctypes.c_double)]


class _Stats(ctypes.Structure):
    _fields_ = [("overflow", ctypes.c_uint32), ("reserved", ctypes.c_uint32), ("sumsq", ctypes.c_double)]


_p = ctypes.c_void_p
_lib.zero_host_adam_step.argtypes = [_p, ctypes.c_int32, ctypes.c_double, _p, _p, _p, _p, ctypes.c_int64,
                                     ctypes.c_int64, ctypes.POINTER(_HParams), ctypes.POINTER(_Stats),
                                     ctypes.c_int32, ctypes.c_int32]
_lib.zero_host_adam_step.restype = ctypes.c_int
_lib.zero_host_adam_set_isa.argtypes = [ctypes.c_int32]
_lib.zero_host_adam_set_isa.restype = ctypes.c_int
_lib.zero_host_last_error.argtypes = []
_lib.zero_host_last_error.restype = ctypes.c_char_p


class HostAdamError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"host Adam error {status}: {message}")
        self.status = status


def library() -> ctypes.CDLL:
    return _lib


def set_isa(level: int = 0) -> int:
    """Instruction set level for later calls (0 = best); returns the level used."""
    r = _lib.zero_host_adam_set_isa(int(level))
    if r < 0:
        raise HostAdamError(r, _lib.zero_host_last_error().decode())
    return r


def _arr(a, dtype, name, n=None):
    if not isinstance(a, np.ndarray) or a.dtype != dtype or not a.flags.c_contiguous:
        raise TypeError(f"{name} must be a C-contiguous numpy {np.dtype(dtype)} array")
    if n is not None and a.size != n:
        raise ValueError(f"{name} has {a.size} elements, expected {n}")
    return a.ctypes.data


def adam_step(grad, master, exp_avg, exp_avg_sq, param16, *, step: int, lr: float, betas=(0.9, 0.999),
              eps: float = 1e-8, inv_grad_scale: float = 1.0, max_grad_norm: float = 0.0, stats=None,
              threads: int = 0) -> tuple[int, float]:
    """The whole shard step in place on host arrays (grad uint16 fp16 bits or
    float32; states float32; param16 uint16).  ``stats`` = (overflow, sumsq)
    precomputed (e.g. all-reduced), else computed here.  Returns the
    (overflow, sumsq) the step used."""
    n = master.size
    if grad.dtype == np.uint16:
        dt = F16
    elif grad.dtype == np.float32:
        dt = F32
    else:
        raise TypeError("grad must be uint16 (fp16 bits) or float32")
    ptrs = [_arr(grad, grad.dtype, "grad", n), _arr(master, np.float32, "master", n),
            _arr(exp_avg, np.float32, "exp_avg", n), _arr(exp_avg_sq, np.float32, "exp_avg_sq", n),
            _arr(param16, np.uint16, "param16", n)]
    hp = _HParams(float(lr), float(betas[0]), float(betas[1]), float(eps), float(max_grad_norm))
    st = _Stats(0, 0, 0.0)
    pre = 0
    if stats is not None:
        st.overflow, st.sumsq, pre = int(stats[0]), float(stats[1]), 1
    r = _lib.zero_host_adam_step(ptrs[0], dt, float(inv_grad_scale), *ptrs[1:], n, int(step), ctypes.byref(hp),
                                 ctypes.byref(st), pre, int(threads))
    if r != 0:
        raise HostAdamError(r, _lib.zero_host_last_error().decode())
    return int(st.overflow), float(st.sumsq)
