"""ctypes binding of libzero_shard.so (include/zero_shard.h).

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  PyTorch supplies device memory and the current HIP stream.  If the
library has not been built this module raises at import, so no call can fall
back to another implementation.
"""
from __future__ import annotations

import ctypes
import os
import struct
from typing import NamedTuple, Sequence

from . import build as _build

# ZERO_SHARD_LIBRARY names another build of the same library (for example
# one with the host code under a sanitizer); by default the in-tree build.
LIB_PATH = os.environ.get("ZERO_SHARD_LIBRARY") or _build.library_path("libzero_shard.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build the HIP library first "
        "(python zero_partitioned_mixed_flat_amd/build.py)")

# PyTorch ships its own HIP runtime (SONAME libamdhip64.so.7).  Loading torch
# first makes this library bind to that same runtime; loading it first would
# bring a second HIP runtime into the process, which then finds no device.
import torch  # noqa: E402,F401

_lib = ctypes.CDLL(LIB_PATH)

# the version of include/zero_shard.h this binding is written against
ZERO_SHARD_ABI_VERSION = 7
_lib.zero_shard_abi_version.argtypes = []
_lib.zero_shard_abi_version.restype = ctypes.c_int
if _lib.zero_shard_abi_version() != ZERO_SHARD_ABI_VERSION:
    raise ImportError(
        f"{LIB_PATH} implements ABI version {_lib.zero_shard_abi_version()}, this binding needs "
        f"{ZERO_SHARD_ABI_VERSION}: rebuild it (python zero_partitioned_mixed_flat_amd/build.py)")

ZERO_OK = 0
ZERO_ERR_INVALID_ARG = -1
ZERO_ERR_MISALIGNED = -2
ZERO_ERR_WORKSPACE = -3
ZERO_ERR_HIP = -4
ZERO_ERR_INT_OVERFLOW = -5
ZERO_F16 = 1
ZERO_F32 = 2
ZERO_MAX_SLICES = 64
ZERO_QWZ_BLOCK = 256
ZERO_NOALLOC_SCRATCH_BYTES = 32768
STATS_BYTES = 16


class _Layout(ctypes.Structure):
    _fields_ = [("psi", ctypes.c_int64), ("psi_padded", ctypes.c_int64),
                ("shard_len", ctypes.c_int64), ("offset", ctypes.c_int64),
                ("real_len", ctypes.c_int64)]


class _HParams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_double), ("beta1", ctypes.c_double),
                ("beta2", ctypes.c_double), ("eps", ctypes.c_double),
                ("max_grad_norm", ctypes.c_double)]


_p = ctypes.c_void_p
_i32, _i64, _dbl, _sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_double, ctypes.c_size_t

_lib.zero_partition_layout.argtypes = [_i64, _i32, _i32, _i64, ctypes.POINTER(_Layout)]
_lib.zero_partition_layout.restype = ctypes.c_int
_lib.zero_model_state_bytes.argtypes = [_dbl, _i32, _i32, _dbl, ctypes.POINTER(_dbl)]
_lib.zero_model_state_bytes.restype = ctypes.c_int
_lib.zero_workspace_bytes.argtypes = [_i64]
_lib.zero_workspace_bytes.restype = _sz
_lib.zero_shard_grad_reduce.argtypes = [_p, _i32, _i64, _p, _p, _dbl, _p, _sz, _p]
_lib.zero_shard_grad_reduce.restype = ctypes.c_int
_lib.zero_shard_allgather.argtypes = [_p, _i32, _i64, _i64, _p, _p]
_lib.zero_shard_allgather.restype = ctypes.c_int
_lib.zero_shard_grad_stats.argtypes = [_p, ctypes.c_int, _i64, _dbl, _p, _p, _sz, _p]
_lib.zero_shard_grad_stats.restype = ctypes.c_int
_lib.zero_shard_adam_step.argtypes = [_p, ctypes.c_int, _dbl, _p, _p, _p, _p, _i64, _i64,
                                      ctypes.POINTER(_HParams), _p, _i32, _p, _sz, _p]
_lib.zero_shard_adam_step.restype = ctypes.c_int
_lib.zero_shard_adam_step_qwz.argtypes = [_p, ctypes.c_int, _dbl, _p, _p, _p, _p, _p, _p, _i64, _i64,
                                          ctypes.POINTER(_HParams), _p, _i32, _p, _sz, _p]
_lib.zero_shard_adam_step_qwz.restype = ctypes.c_int
_lib.zero_shard_adam_step_device_t.argtypes = [_p, ctypes.c_int, _dbl, _p, _p, _p, _p, _p, _p, _i64, _p,
                                               ctypes.POINTER(_HParams), _p, _i32, _p, _sz, _p]
_lib.zero_shard_adam_step_device_t.restype = ctypes.c_int
_lib.zero_shard_adam_step_noalloc.argtypes = [_p, ctypes.c_int, _dbl, _p, _p, _p, _p, _i64, _i64,
                                              ctypes.POINTER(_HParams), _p, _i32, _p]
_lib.zero_shard_adam_step_noalloc.restype = ctypes.c_int
_lib.zero_qwz_quantize.argtypes = [_p, _i64, _p, _p, _p]
_lib.zero_qwz_quantize.restype = ctypes.c_int
_lib.zero_qwz_allgather.argtypes = [_p, _p, _i32, _i64, _i64, _p, _p]
_lib.zero_qwz_allgather.restype = ctypes.c_int
_lib.zero_status_string.argtypes = [ctypes.c_int]
_lib.zero_status_string.restype = ctypes.c_char_p
_lib.zero_last_error.argtypes = []
_lib.zero_last_error.restype = ctypes.c_char_p


def library() -> ctypes.CDLL:
    return _lib


class ZeroError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_lib.zero_status_string(status).decode()} ({status}): {message}")
        self.status = status


def _check(status: int) -> None:
    if status != ZERO_OK:
        raise ZeroError(status, _lib.zero_last_error().decode())


class Layout(NamedTuple):
    psi: int
    psi_padded: int
    shard_len: int
    offset: int
    real_len: int


def partition_layout(psi: int, n_ranks: int, rank: int, align: int = 128) -> Layout:
    out = _Layout()
    _check(_lib.zero_partition_layout(psi, n_ranks, rank, align, ctypes.byref(out)))
    return Layout(out.psi, out.psi_padded, out.shard_len, out.offset, out.real_len)


def model_state_bytes(psi: float, n_ranks: int, stage: int, K: float = 12.0) -> float:
    out = ctypes.c_double()
    _check(_lib.zero_model_state_bytes(psi, n_ranks, stage, K, ctypes.byref(out)))
    return out.value


def workspace_bytes(length: int) -> int:
    return int(_lib.zero_workspace_bytes(length))


# ------------------------------------------------------------ tensor plumbing
def _torch():
    import torch
    return torch


def _stream(stream) -> int:
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return int(s.cuda_stream)


def _dev_ptr(t, dtype, name: str, numel: int | None = None) -> int:
    torch = _torch()
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, expected {numel}")
    return t.data_ptr()


def new_stats(device=None):
    """A device buffer for one zero_grad_stats_t (16 bytes)."""
    torch = _torch()
    return torch.zeros(STATS_BYTES, dtype=torch.uint8, device=device or "cuda")


def read_stats(stats) -> tuple[int, float]:
    """(overflow, sumsq) from a stats buffer; synchronises with the device."""
    raw = bytes(stats.cpu().numpy().tobytes())
    overflow, _reserved, sumsq = struct.unpack("<IId", raw[:STATS_BYTES])
    return overflow, sumsq


def new_workspace(length: int, device=None):
    torch = _torch()
    return torch.empty(max(workspace_bytes(length), 16), dtype=torch.uint8, device=device or "cuda")


def _temp_workspace(length: int, device, stream):
    """A workspace for one call.  It is freed when the call returns, while
    the kernels may still use it on `stream`; recording that stream keeps the
    caching allocator from handing the block to another allocation until the
    stream has passed this point."""
    ws = new_workspace(length, device)
    if stream is not None:
        ws.record_stream(stream)
    return ws


def _grad_dtype(grad) -> int:
    torch = _torch()
    if grad.dtype == torch.float16:
        return ZERO_F16
    if grad.dtype == torch.float32:
        return ZERO_F32
    raise TypeError("grad must be float16 or float32")


def grad_reduce(slices: Sequence, out, *, stats=None, inv_grad_scale: float = 1.0,
                workspace=None, stream=None) -> None:
    """out[j] = sum over r of slices[r][j] in fp32, rank order; with
    ``stats`` also the overflow flag and sum of squares of out*inv_grad_scale."""
    torch = _torch()
    n = len(slices)
    if not 1 <= n <= ZERO_MAX_SLICES:
        raise ValueError(f"need 1..{ZERO_MAX_SLICES} slices, got {n}")
    length = out.numel()
    ptrs = (ctypes.c_void_p * n)(*[_dev_ptr(s, torch.float16, f"slices[{i}]", length)
                                   for i, s in enumerate(slices)])
    out_p = _dev_ptr(out, torch.float32, "out")
    stats_p = ws_p = None
    ws_n = 0
    if stats is not None:
        stats_p = _dev_ptr(stats, None, "stats")
        if workspace is None:
            workspace = _temp_workspace(length, out.device, stream)
        ws_p, ws_n = _dev_ptr(workspace, None, "workspace"), workspace.numel() * workspace.element_size()
    _check(_lib.zero_shard_grad_reduce(ctypes.cast(ptrs, ctypes.c_void_p), n, length, out_p, stats_p,
                                       float(inv_grad_scale), ws_p, ws_n, _stream(stream)))


def allgather(shards: Sequence, replica, *, stream=None) -> None:
    """replica (fp16, psi elements) = the shards (fp16, equal lengths, rank
    order) concatenated without the padding beyond psi."""
    torch = _torch()
    n = len(shards)
    if not 1 <= n <= ZERO_MAX_SLICES:
        raise ValueError(f"need 1..{ZERO_MAX_SLICES} shards, got {n}")
    shard_len = shards[0].numel()
    ptrs = (ctypes.c_void_p * n)(*[_dev_ptr(s, torch.float16, f"shards[{i}]", shard_len)
                                   for i, s in enumerate(shards)])
    _check(_lib.zero_shard_allgather(ctypes.cast(ptrs, ctypes.c_void_p), n, shard_len, replica.numel(),
                                     _dev_ptr(replica, torch.float16, "replica"), _stream(stream)))


def grad_stats(grad, stats, *, inv_grad_scale: float, workspace=None, stream=None) -> None:
    length = grad.numel()
    g_p = _dev_ptr(grad, None, "grad")
    if workspace is None:
        workspace = _temp_workspace(length, grad.device, stream)
    _check(_lib.zero_shard_grad_stats(g_p, _grad_dtype(grad), length, float(inv_grad_scale),
                                      _dev_ptr(stats, None, "stats"), _dev_ptr(workspace, None, "workspace"),
                                      workspace.numel() * workspace.element_size(), _stream(stream)))


def adam_step(grad, master, exp_avg, exp_avg_sq, param16, *, step: int, lr: float,
              betas=(0.9, 0.999), eps: float = 1e-8, inv_grad_scale: float = 1.0,
              max_grad_norm: float = 0.0, stats, stats_precomputed: bool = False,
              workspace=None, qwz_codes=None, qwz_scales=None, stream=None) -> None:
    """One rank's fused Adam step on its shard, in place (see zero_shard.h);
    max_grad_norm > 0 clips to that global 2-norm using stats->sumsq.  With
    qwz_codes (int8 [len]) and qwz_scales (fp32 [qwz_scales_len(len)]) the
    fresh fp16 shard is also block-INT8 encoded in the same pass."""
    torch = _torch()
    length = master.numel()
    g_p = _dev_ptr(grad, None, "grad", length)
    ptrs = [_dev_ptr(master, torch.float32, "master", length),
            _dev_ptr(exp_avg, torch.float32, "exp_avg", length),
            _dev_ptr(exp_avg_sq, torch.float32, "exp_avg_sq", length),
            _dev_ptr(param16, torch.float16, "param16", length)]
    hp = _HParams(float(lr), float(betas[0]), float(betas[1]), float(eps), float(max_grad_norm))
    ws_p, ws_n = None, 0
    if not stats_precomputed:
        if workspace is None:
            workspace = _temp_workspace(length, master.device, stream)
        ws_p, ws_n = _dev_ptr(workspace, None, "workspace"), workspace.numel() * workspace.element_size()
    tail = (length, int(step), ctypes.byref(hp), _dev_ptr(stats, None, "stats"), int(bool(stats_precomputed)),
            ws_p, ws_n, _stream(stream))
    if (qwz_codes is None) != (qwz_scales is None):
        raise ValueError("qwz_codes and qwz_scales go together")
    if qwz_codes is None:
        _check(_lib.zero_shard_adam_step(g_p, _grad_dtype(grad), float(inv_grad_scale), *ptrs, *tail))
    else:
        q = [_dev_ptr(qwz_codes, torch.int8, "qwz_codes", length),
             _dev_ptr(qwz_scales, torch.float32, "qwz_scales", qwz_scales_len(length))]
        _check(_lib.zero_shard_adam_step_qwz(g_p, _grad_dtype(grad), float(inv_grad_scale), *ptrs, *q, *tail))


def adam_step_noalloc(grad, master, exp_avg, exp_avg_sq, param16, *, step: int, lr: float,
                      betas=(0.9, 0.999), eps: float = 1e-8, inv_grad_scale: float = 1.0,
                      max_grad_norm: float = 0.0, stats, stats_precomputed: bool = False, stream=None) -> None:
    """adam_step without a workspace: the statistics' partials go to the
    library's static per-device scratch (zero_shard_adam_step_noalloc), so
    the call allocates nothing.  Calls on one device must not overlap in
    time (they share that scratch)."""
    torch = _torch()
    length = master.numel()
    g_p = _dev_ptr(grad, None, "grad", length)
    ptrs = [_dev_ptr(master, torch.float32, "master", length),
            _dev_ptr(exp_avg, torch.float32, "exp_avg", length),
            _dev_ptr(exp_avg_sq, torch.float32, "exp_avg_sq", length),
            _dev_ptr(param16, torch.float16, "param16", length)]
    hp = _HParams(float(lr), float(betas[0]), float(betas[1]), float(eps), float(max_grad_norm))
    _check(_lib.zero_shard_adam_step_noalloc(g_p, _grad_dtype(grad), float(inv_grad_scale), *ptrs, length,
                                             int(step), ctypes.byref(hp), _dev_ptr(stats, None, "stats"),
                                             int(bool(stats_precomputed)), _stream(stream)))


def new_step_counter(device=None):
    """A device zero_step_counter_t (16 bytes, held as two int64): the count
    of applied steps, starting at 0, and the bias corrections of the last
    call."""
    torch = _torch()
    return torch.zeros(2, dtype=torch.int64, device=device or "cuda")


def read_step_counter(counter) -> int:
    """The number of steps a device step counter has counted (synchronises)."""
    return int(counter[0].item())


def adam_step_device_t(grad, master, exp_avg, exp_avg_sq, param16, *, applied_steps, lr: float,
                       betas=(0.9, 0.999), eps: float = 1e-8, inv_grad_scale: float = 1.0,
                       max_grad_norm: float = 0.0, stats, stats_precomputed: bool = False, workspace=None,
                       qwz_codes=None, qwz_scales=None, stream=None) -> None:
    """adam_step with the step number in device memory: t = applied_steps + 1,
    and applied_steps is advanced on the device only when the step applies,
    so the call can be captured in a graph and replayed every step."""
    torch = _torch()
    length = master.numel()
    g_p = _dev_ptr(grad, None, "grad", length)
    ptrs = [_dev_ptr(master, torch.float32, "master", length),
            _dev_ptr(exp_avg, torch.float32, "exp_avg", length),
            _dev_ptr(exp_avg_sq, torch.float32, "exp_avg_sq", length),
            _dev_ptr(param16, torch.float16, "param16", length)]
    if (qwz_codes is None) != (qwz_scales is None):
        raise ValueError("qwz_codes and qwz_scales go together")
    q = [None, None]
    if qwz_codes is not None:
        q = [_dev_ptr(qwz_codes, torch.int8, "qwz_codes", length),
             _dev_ptr(qwz_scales, torch.float32, "qwz_scales", qwz_scales_len(length))]
    hp = _HParams(float(lr), float(betas[0]), float(betas[1]), float(eps), float(max_grad_norm))
    ws_p, ws_n = None, 0
    if not stats_precomputed:
        if workspace is None:
            workspace = _temp_workspace(length, master.device, stream)
        ws_p, ws_n = _dev_ptr(workspace, None, "workspace"), workspace.numel() * workspace.element_size()
    _check(_lib.zero_shard_adam_step_device_t(g_p, _grad_dtype(grad), float(inv_grad_scale), *ptrs, *q, length,
                                              _dev_ptr(applied_steps, torch.int64, "applied_steps", 2),
                                              ctypes.byref(hp), _dev_ptr(stats, None, "stats"),
                                              int(bool(stats_precomputed)), ws_p, ws_n, _stream(stream)))


def qwz_scales_len(length: int) -> int:
    """Number of qwZ blocks (one fp32 scale each) of `length` values."""
    return -(-int(length) // ZERO_QWZ_BLOCK)


def qwz_quantize(x16, codes, scales, *, stream=None) -> None:
    """Block-INT8 encoding of fp16 x16 into codes (int8) and scales (fp32)."""
    torch = _torch()
    length = x16.numel()
    _check(_lib.zero_qwz_quantize(_dev_ptr(x16, torch.float16, "x16"), length,
                                  _dev_ptr(codes, torch.int8, "codes", length),
                                  _dev_ptr(scales, torch.float32, "scales", qwz_scales_len(length)),
                                  _stream(stream)))


def qwz_allgather(codes: Sequence, scales: Sequence, replica, *, stream=None) -> None:
    """replica (fp16, psi elements) = the decoded shards (int8 codes and fp32
    scales per rank, rank order) concatenated without the padding."""
    torch = _torch()
    n = len(codes)
    if not 1 <= n <= ZERO_MAX_SLICES or len(scales) != n:
        raise ValueError(f"need 1..{ZERO_MAX_SLICES} code and scale buffers, got {n} and {len(scales)}")
    shard_len = codes[0].numel()
    cp = (ctypes.c_void_p * n)(*[_dev_ptr(c, torch.int8, f"codes[{i}]", shard_len) for i, c in enumerate(codes)])
    sp = (ctypes.c_void_p * n)(*[_dev_ptr(s, torch.float32, f"scales[{i}]", qwz_scales_len(shard_len))
                                 for i, s in enumerate(scales)])
    _check(_lib.zero_qwz_allgather(ctypes.cast(cp, ctypes.c_void_p), ctypes.cast(sp, ctypes.c_void_p), n, shard_len,
                                   replica.numel(), _dev_ptr(replica, torch.float16, "replica"), _stream(stream)))
