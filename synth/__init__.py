"""Seeded synthetic inputs for batch-invariant paged attention (and RMSNorm and GEMM).

This package generates inputs only: token values, page placements, batches and the
mixed continuous-batching schedule. It holds none of the attention arithmetic, so the
fp64 oracle checks and the GPU path can share it without sharing any of the method.
"""

from .workloads import (  # noqa: F401
    AttnShape,
    Batch,
    SeqSpec,
    bf16_round,
    bf16_bits,
    from_bf16_bits,
    token_values,
    build_batch,
    poisoned_pool,
    mixed_trace,
    TraceStep,
    Trace,
    PageAllocator,
    CONFIG_SHAPES,
    norm_inputs,
    gemm_inputs,
)
