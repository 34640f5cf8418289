"""Oracle helper: interpret bfloat16 bit patterns.  TEST INFRASTRUCTURE ONLY.

NumPy has no bfloat16 type, so bf16 activations travel as uint16 bit patterns.
A bf16 value is the upper half of the fp32 with the same bits, so widening is
a 16-bit left shift and is exact.
"""

import numpy as np


def bf16_bits_to_f32(bits):
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)
