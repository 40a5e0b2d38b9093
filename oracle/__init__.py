"""CPU oracle for exact softmax attention (float64 NumPy).

Test infrastructure only: the test suite, the smoke check and the CPU
baseline leg of the benchmark use it. The GPU library never imports it.
"""
from .dense import (MASKS, NA2D, NA3D, allowed, attention, attention_backward, masked_attention,
                    masked_attention_backward, probs)

__all__ = ["NA2D", "NA3D", "MASKS", "allowed", "attention", "attention_backward", "masked_attention",
           "masked_attention_backward", "probs"]
