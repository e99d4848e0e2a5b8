"""How the oracle reads its inputs: storage bits to exact float64.

bfloat16 is the top half of an IEEE binary32, so widening ``bits << 16`` to
float32 and then to float64 is exact.  float32 inputs widen exactly too.

Test infrastructure only (see the package docstring).
"""

from __future__ import annotations

import numpy as np


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def to_f64(x: np.ndarray) -> np.ndarray:
    """uint16 arrays are bf16 bit patterns; float arrays widen as they are."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return bf16_to_f64(x)
    return x.astype(np.float64)
