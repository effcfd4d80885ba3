"""fp64 CPU oracle for attention (test infrastructure only).

Only tests, the smoke check and the CPU-baseline leg of the benchmark import
this package. The HIP library never does, and this package imports nothing
from it.
"""
from .attention import (MaskSpec, attention_bwd, attention_bwd_head, attention_dq_rows, attention_fwd,
                        attention_probs, attention_rows, mask_matrix)

__all__ = ["MaskSpec", "attention_fwd", "attention_bwd", "attention_bwd_head", "attention_dq_rows",
           "attention_probs", "attention_rows", "mask_matrix"]
