"""Oracle helper: rounding to the stored bf16 precision (float64 in and out).

Test infrastructure only (see the package docstring).
"""

import numpy as np


def round_bf16(x):
    """float64 -> float32 -> nearest bf16 value (ties to even), as float64: the
    rounding a value held in fp32 on the device gets when it is stored as bf16."""
    f = np.asarray(x, np.float64).astype(np.float32)
    b = f.view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000
    return b.astype(np.uint32).view(np.float32).astype(np.float64)
