"""CPU fp64 oracle for Cut Cross-Entropy: test infrastructure only.

Only tests/, the smoke check and the benchmark's CPU-baseline leg may import
this package; the product path never does.
"""
from .cce_oracle import (  # noqa: F401
    FILTER_LOG_THRESHOLD, Backward, Forward, G_columns, backward, dC_rows, db_rows, dE_rows, filter_keep,
    forward, grad_scale, logits, lse_all, lse_and_keep, lse_keep_nll, reduce_loss, row_logsumexp,
    soft_target_rows, softmax_grad_rows, tile_blocks, tile_row_max, valid_rows,
)
