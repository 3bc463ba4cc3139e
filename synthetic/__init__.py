"""Seeded synthetic inputs for speculative-decoding verify attention.

This package only generates data: query rows, paged K/V pools (fp32, fp16 or
8-bit blocks with fp16 scales), block tables, context lengths and parent
arrays.  It holds none of the attention arithmetic, so both the fp64 oracle
and the HIP path can consume its arrays without sharing any code.
"""

from .workloads import (  # noqa: F401
    PAGE,
    Workload,
    bf16_bits_from_f32,
    bf16_bits_to_f32,
    make_workload,
    tree_parent,
    tiny_dense,
    qwen_dense,
    q8_long,
    paged_ragged,
    tree_mixed,
    chain,
    chain_parent,
    mixed_lowering,
    new_kv_rows,
    peaked,
    rising_max,
    late_dominant,
)
