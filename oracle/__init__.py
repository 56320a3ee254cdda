"""CPU float64 oracle for exact softmax attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or links
anything here; only the tests, the smoke check and the benchmark's CPU baseline
leg use it.  It shares no code with the HIP kernels.
"""
from .exact import (
    attention,
    attention_rows,
    causal_mask,
    compressed_causal_mask,
    log_sum_exp,
    logits,
    probabilities,
    row_log_sum_exp,
    softmax_rows,
    weighted_values,
    window_mask,
)

__all__ = [
    "attention",
    "attention_rows",
    "causal_mask",
    "compressed_causal_mask",
    "log_sum_exp",
    "logits",
    "probabilities",
    "row_log_sum_exp",
    "softmax_rows",
    "weighted_values",
    "window_mask",
]
