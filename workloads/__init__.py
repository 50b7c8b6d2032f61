"""Seeded synthetic inputs for paged grouped-query attention (head_dim 256).

This package only draws inputs: lengths, Q, the paged K/V pool, block tables
and sparse index lists.  It holds none of the attention arithmetic, so both
the fp64 oracle and the HIP library can consume the same inputs without
sharing any code path.
"""
from .synth import (  # noqa: F401
    Problem, BF16, FP8, NAN_CODE, config, config_names, make_causal, make_sparse, make_prefill_quant,
    poison_unused, visible_pairs, kv_bytes_read, gathered_bytes, sample_rows,
)
