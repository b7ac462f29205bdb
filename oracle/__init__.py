"""CPU float64 oracle for the fused LM-head op.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the GPU library or its Python binding.
"""

from .lmhead_ref import (  # noqa: F401
    backward,
    backward_f64,
    backward_shard_f64,
    bf16_to_f64,
    compact,
    forward,
    forward_f64,
    logit_grad,
    logits_input_fwd_bwd,
    merge_shard_partials,
    row_stats,
    rows_fwd_bwd,
    shard_partials_f64,
)
