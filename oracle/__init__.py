"""Float64 CPU oracle for exact attention (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product path never calls it: it shares no code
with the HIP library and imports nothing from it.
"""
from .attention import (attention_forward, attention_partial, attention_rows, attention_varlen, merge_partials,
                        scores_row)
from .backward import attention_backward, attention_varlen_backward

__all__ = ["attention_forward", "attention_rows", "scores_row", "attention_partial", "merge_partials",
           "attention_varlen", "attention_backward", "attention_varlen_backward"]
