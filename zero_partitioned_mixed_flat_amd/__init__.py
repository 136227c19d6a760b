"""MI355X-native per-rank ZeRO shard optimizer step.

One data-parallel rank's share of ZeRO-partitioned mixed-precision training
(the pages "DeepSpeed ZeRO Stages", "ZeRO Stage 1 Math", "ZeRO Optimization:
Stages 1, 2, and 3 Explained", "DeepSpeed ZeRO: Extreme Memory Efficiency"):

* ``partition_layout``  -- the rank's disjoint, padded shard of the flat space
* ``grad_reduce``       -- owner-side fp32 sum of N fp16 gradient slices
* ``grad_stats``        -- overflow flag and sum of squares of the gradient
* ``adam_step``         -- fused fp32 Adam update of master/m/v + fp16 copy
  (``adam_step_device_t``: the same with the step number in device memory;
  ``adam_step_noalloc``: the same without a workspace, for callers that
  cannot allocate)
* ``allgather``         -- the flat fp16 replica from the N owners' shards
* ``qwz_quantize``, ``qwz_allgather``, ``adam_step(qwz_codes=...)`` -- the
  block-INT8 (qwZ) encoding of the fp16 shard and its decoding gather

All device work runs in the HIP library ``libzero_shard.so`` (C ABI in
``include/zero_shard.h``); this package only marshals arguments.
"""
from ._native import (  # noqa: F401
    STATS_BYTES, ZERO_F16, ZERO_F32, ZERO_MAX_SLICES, ZERO_NOALLOC_SCRATCH_BYTES, ZERO_QWZ_BLOCK, Layout,
    ZeroError, adam_step, adam_step_device_t, adam_step_noalloc, allgather, grad_reduce, grad_stats, library,
    model_state_bytes, new_stats, new_step_counter, new_workspace, partition_layout, qwz_allgather, qwz_quantize,
    qwz_scales_len, read_stats, read_step_counter, workspace_bytes)

__all__ = [
    "Layout", "ZeroError", "partition_layout", "model_state_bytes", "workspace_bytes",
    "new_workspace", "new_stats", "read_stats", "grad_reduce", "grad_stats", "adam_step", "allgather",
    "adam_step_device_t", "new_step_counter", "read_step_counter", "adam_step_noalloc",
    "qwz_quantize", "qwz_allgather", "qwz_scales_len",
    "library", "ZERO_F16", "ZERO_F32", "ZERO_MAX_SLICES", "ZERO_QWZ_BLOCK", "ZERO_NOALLOC_SCRATCH_BYTES",
    "STATS_BYTES",
]
