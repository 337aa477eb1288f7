"""CPU oracle (float64 NumPy) for exact attention.

TEST INFRASTRUCTURE ONLY: imported by the tests, the package smoke check and the
benchmark's CPU-baseline leg; never by the product path.
"""
from .attention import (attention_backward, attention_dq_rows, attention_forward, kv_head, softmax_probs,
                        visible_mask)

__all__ = ["attention_forward", "attention_backward", "attention_dq_rows", "kv_head", "softmax_probs",
           "visible_mask"]
