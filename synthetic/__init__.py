"""Seeded synthetic inputs for the attention hot path.

This module only draws random numbers and lays them out; it holds none of
the attention arithmetic.  Both the oracle-side tests and the GPU-side tests
and benchmark take their inputs from here.
"""

from .workloads import (  # noqa: F401
    WORKLOADS,
    tensor_seed,
    normal,
    uniform,
    prefill_inputs,
    chunk_inputs,
    ring_decode_inputs,
    contiguous_decode_inputs,
    kv_scales,
    multi_ring_inputs,
    multi_contiguous_inputs,
    e4m3_codes,
    ring_decode_inputs_fp8,
    contiguous_decode_inputs_fp8,
    decode_positions,
    sparse_selection,
    sparse_inputs,
    sparse_inputs_fp8,
)
