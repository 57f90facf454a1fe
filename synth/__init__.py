"""Seeded synthetic inputs shared by the oracle checks, the GPU tests and the bench.

This package draws random numbers and applies the rotary position embedding
to them; it holds none of the quantization method's arithmetic (no scores,
allocation, codebooks, scales, packing or attention).
"""
from .workloads import (  # noqa: F401
    WORKLOADS,
    Workload,
    rope_frequencies,
    apply_rope,
    block_sigmas,
    seq_block_sigmas,
    gen_layer,
    gen_query,
    to_input_dtype,
)
