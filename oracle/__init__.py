"""ctypes wrapper around the plain C oracle (``zero_oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by the smoke check and by
the CPU-baseline leg of ``bench.py``; never by the product package.  Every
function takes and returns numpy arrays and forwards them unchanged to the
single-threaded C routines; no arithmetic happens here.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "zero_oracle.c")
# ZERO_ORACLE_LIB points the wrapper at another build of the same source; the
# mutation tests use it to load deliberately broken copies of the oracle.
LIBRARY = os.environ.get("ZERO_ORACLE_LIB") or os.path.join(HERE, "liboracle.so")

# The oracle is built without contraction and without fast-math so that each
# float operation is one correctly rounded binary32 operation (SSE on x86-64).
CFLAGS = ["-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math",
          "-fno-strict-aliasing", "-fPIC", "-shared", "-Wall", "-Wextra"]


def build(force: bool = True) -> str:
    """Compile ``zero_oracle.c`` into ``liboracle.so`` with gcc."""
    if force or not os.path.exists(LIBRARY):
        tmp = LIBRARY + ".tmp"
        subprocess.run(["gcc", *CFLAGS, "-o", tmp, SOURCE, "-lm"], check=True)
        os.replace(tmp, LIBRARY)
    return LIBRARY


_lib = None

_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
_u32 = ctypes.c_uint32
_dbl = ctypes.c_double
_ptr = ctypes.c_void_p


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIBRARY):
            build(force=False)
        L = ctypes.CDLL(LIBRARY)
        L.zo_partition_layout.argtypes = [_i64, _i32, _i32, _i64, _ptr]
        L.zo_partition_layout.restype = ctypes.c_int
        L.zo_model_state_bytes.argtypes = [_dbl, _i32, _i32, _dbl]
        L.zo_model_state_bytes.restype = _dbl
        L.zo_f16_to_f32.argtypes = [ctypes.c_uint16]
        L.zo_f16_to_f32.restype = ctypes.c_float
        L.zo_f32_to_f16.argtypes = [ctypes.c_float]
        L.zo_f32_to_f16.restype = ctypes.c_uint16
        for name in ("zo_f16_to_f32_array", "zo_f32_to_f16_array"):
            getattr(L, name).argtypes = [_ptr, _ptr, _i64]
            getattr(L, name).restype = None
        L.zo_grad_reduce.argtypes = [_ptr, _i32, _i64, _ptr]
        L.zo_grad_reduce.restype = None
        L.zo_allgather.argtypes = [_ptr, _i32, _i64, _i64, _ptr]
        L.zo_allgather.restype = None
        L.zo_qwz_quantize.argtypes = [_ptr, _i64, _ptr, _ptr]
        L.zo_qwz_quantize.restype = None
        L.zo_qwz_dequantize.argtypes = [_ptr, _ptr, _i64, _ptr]
        L.zo_qwz_dequantize.restype = None
        for name in ("zo_grad_stats_f16", "zo_grad_stats_f32"):
            getattr(L, name).argtypes = [_ptr, _i64, _dbl, _ptr, _ptr]
            getattr(L, name).restype = None
        L.zo_adam_scalars.argtypes = [_dbl, _dbl, _dbl, _dbl, _dbl, _i64, _ptr]
        L.zo_adam_scalars.restype = ctypes.c_int
        L.zo_adam_element.argtypes = [ctypes.c_float, _ptr, _ptr, _ptr, _ptr, _ptr]
        L.zo_adam_element.restype = None
        for name in ("zo_adam_apply_f16", "zo_adam_apply_f32"):
            getattr(L, name).argtypes = [_ptr, _ptr, _ptr, _ptr, _ptr, _i64, _i64,
                                         _dbl, _dbl, _dbl, _dbl, _dbl, _u32]
            getattr(L, name).restype = ctypes.c_int
        for name in ("zo_shard_adam_step_f16", "zo_shard_adam_step_f32"):
            getattr(L, name).argtypes = [_ptr, _ptr, _ptr, _ptr, _ptr, _i64, _i64,
                                         _dbl, _dbl, _dbl, _dbl, _dbl, _dbl, _ptr, _ptr]
            getattr(L, name).restype = ctypes.c_int
        L.zo_clip_factor.argtypes = [_dbl, _dbl]
        L.zo_clip_factor.restype = _dbl
        _lib = L
    return _lib


def _p(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be contiguous"
    return a.ctypes.data


def _need(a: np.ndarray, dtype) -> np.ndarray:
    if a.dtype != dtype or not a.flags["C_CONTIGUOUS"]:
        raise TypeError(f"expected a contiguous {np.dtype(dtype)} array, got {a.dtype}")
    return a


# --------------------------------------------------------------------- layout
def partition_layout(psi: int, n_ranks: int, rank: int, align: int = 128):
    """Returns (status, (psi, psi_padded, shard_len, offset, real_len))."""
    out = np.zeros(5, dtype=np.int64)
    st = lib().zo_partition_layout(psi, n_ranks, rank, align, _p(out))
    return st, tuple(int(x) for x in out)


def model_state_bytes(psi: float, n_ranks: int, stage: int, K: float = 12.0) -> float:
    return lib().zo_model_state_bytes(psi, n_ranks, stage, K)


# ------------------------------------------------------------------ binary16
def f16_to_f32(bits: np.ndarray) -> np.ndarray:
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(bits.shape, dtype=np.float32)
    lib().zo_f16_to_f32_array(_p(bits), _p(out), bits.size)
    return out


def f32_to_f16(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().zo_f32_to_f16_array(_p(x), _p(out), x.size)
    return out


# --------------------------------------------------------------------- reduce
def grad_reduce(slices) -> np.ndarray:
    """Left fold in rank order; ``slices`` is a list of uint16 arrays or a
    2-D uint16 array of shape [N, len]."""
    rows = [_need(np.asarray(s), np.uint16) for s in slices]
    n = len(rows)
    length = rows[0].size
    assert all(r.size == length for r in rows)
    ptrs = (ctypes.c_void_p * n)(*[_p(r) for r in rows])
    out = np.empty(length, dtype=np.float32)
    lib().zo_grad_reduce(ctypes.cast(ptrs, ctypes.c_void_p), n, length, _p(out))
    return out


# ----------------------------------------------------------------- all-gather
def allgather(shards, psi: int) -> np.ndarray:
    """Flat fp16 replica (uint16 bits, psi elements) from equal-length shards."""
    rows = [_need(np.asarray(s), np.uint16) for s in shards]
    n = len(rows)
    length = rows[0].size
    assert all(r.size == length for r in rows) and psi <= n * length
    ptrs = (ctypes.c_void_p * n)(*[_p(r) for r in rows])
    out = np.empty(psi, dtype=np.uint16)
    lib().zo_allgather(ctypes.cast(ptrs, ctypes.c_void_p), n, length, psi, _p(out))
    return out


# ------------------------------------------------------------------------ qwZ
QWZ_BLOCK = 256


def qwz_quantize(x16: np.ndarray):
    """(codes int8[len], scales float32[ceil(len/256)]) of fp16 bits."""
    x16 = _need(np.ascontiguousarray(x16), np.uint16)
    codes = np.empty(x16.size, dtype=np.int8)
    scales = np.empty(-(-x16.size // QWZ_BLOCK), dtype=np.float32)
    lib().zo_qwz_quantize(_p(x16), x16.size, _p(codes), _p(scales))
    return codes, scales


def qwz_dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    codes = _need(np.ascontiguousarray(codes), np.int8)
    scales = _need(np.ascontiguousarray(scales), np.float32)
    assert scales.size == -(-codes.size // QWZ_BLOCK)
    out = np.empty(codes.size, dtype=np.uint16)
    lib().zo_qwz_dequantize(_p(codes), _p(scales), codes.size, _p(out))
    return out


# ---------------------------------------------------------------------- stats
def grad_stats(grad: np.ndarray, inv_scale: float):
    """Returns (overflow, sumsq) for fp16 bits (uint16) or fp32 gradients."""
    flag = np.zeros(1, dtype=np.uint32)
    ssq = np.zeros(1, dtype=np.float64)
    if grad.dtype == np.uint16:
        lib().zo_grad_stats_f16(_p(_need(grad, np.uint16)), grad.size, inv_scale, _p(flag), _p(ssq))
    else:
        lib().zo_grad_stats_f32(_p(_need(grad, np.float32)), grad.size, inv_scale, _p(flag), _p(ssq))
    return int(flag[0]), float(ssq[0])


# ----------------------------------------------------------------------- Adam
def adam_scalars(lr, beta1, beta2, eps, inv_scale, step):
    s = np.zeros(9, dtype=np.float32)
    st = lib().zo_adam_scalars(lr, beta1, beta2, eps, inv_scale, step, _p(s))
    return st, s


def adam_apply(grad, master, m, v, p16, *, step, lr, beta1, beta2, eps,
               inv_scale, overflow) -> int:
    """In-place gated update of (master, m, v, p16); grad is uint16 fp16 bits
    or float32.  Returns the oracle status code."""
    for a, dt in ((master, np.float32), (m, np.float32), (v, np.float32), (p16, np.uint16)):
        _need(a, dt)
    n = master.size
    assert m.size == n and v.size == n and p16.size == n and grad.size == n
    fn = lib().zo_adam_apply_f16 if grad.dtype == np.uint16 else lib().zo_adam_apply_f32
    if grad.dtype != np.uint16:
        _need(grad, np.float32)
    return fn(_p(grad), _p(master), _p(m), _p(v), _p(p16), n, step, lr, beta1,
              beta2, eps, inv_scale, int(overflow))


def clip_factor(sumsq: float, max_norm: float) -> float:
    return lib().zo_clip_factor(sumsq, max_norm)


def shard_adam_step(grad, master, m, v, p16, *, step, lr, beta1, beta2, eps,
                    inv_scale, max_norm=0.0):
    """Statistics then the gated (and, with max_norm > 0, clipped) update, in
    place.  Returns (status, overflow, sumsq)."""
    for a, dt in ((master, np.float32), (m, np.float32), (v, np.float32), (p16, np.uint16)):
        _need(a, dt)
    n = master.size
    assert m.size == n and v.size == n and p16.size == n and grad.size == n
    flag = np.zeros(1, dtype=np.uint32)
    ssq = np.zeros(1, dtype=np.float64)
    if grad.dtype == np.uint16:
        fn = lib().zo_shard_adam_step_f16
    else:
        _need(grad, np.float32)
        fn = lib().zo_shard_adam_step_f32
    st = fn(_p(grad), _p(master), _p(m), _p(v), _p(p16), n, step, lr, beta1,
            beta2, eps, inv_scale, max_norm, _p(flag), _p(ssq))
    return st, int(flag[0]), float(ssq[0])
