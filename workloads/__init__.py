"""Seeded synthetic inputs for route-sparse GQA attention.

This package draws inputs only: random Q/K/V rounded to bfloat16 bit
patterns, and route-ID tensors with the structure of the layouts the
route-sparse GQA pages describe (right-padded batches, packed THD rows,
a context-parallel query slice against global K/V, a long sequence whose
membership table needs 64-bit offsets).  It holds none of the method's
arithmetic: no validation, deduplication or attention.  Both the CPU
oracle and the HIP path consume exactly the same arrays.
"""

from .generators import (  # noqa: F401
    SELECT_WORKLOADS,
    WORKLOADS,
    SelectWorkload,
    Workload,
    bf16_bits_to_float32,
    float32_to_bf16_bits,
    make_dout,
    make_inputs,
    make_qkv,
    make_routes,
    make_select_inputs,
    random_dout,
    random_select_case,
)
