"""Exact widening of the step's storage types to float64.  Test infrastructure.

bfloat16 values travel as their raw 16-bit patterns (numpy has no bfloat16).
A bfloat16 is the top half of an IEEE float32, so shifting the pattern into
the high 16 bits of a 32-bit word and reinterpreting gives the float32 with
the same value; float32 -> float64 is exact.

Pinned in tests/test_oracle_dtypes.py against hand-checked bit patterns
(1.0, -2.0, the smallest normal, infinities) and against torch's own
bfloat16 -> float64 conversion.
"""

import numpy as np


def bf16_bits_to_f64(bits):
    """Return float64 values of an array of bfloat16 bit patterns (uint16)."""
    b = np.asarray(bits, dtype=np.uint16)
    f32 = (b.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return f32.astype(np.float64)


def to_f64(arr, dtype):
    """Widen ``arr`` stored as ``dtype`` ("bf16" bit patterns or "f32") to float64."""
    if dtype == "bf16":
        return bf16_bits_to_f64(arr)
    if dtype == "f32":
        return np.asarray(arr, dtype=np.float32).astype(np.float64)
    if dtype == "f64":
        return np.asarray(arr, dtype=np.float64)
    raise ValueError(f"unknown storage dtype {dtype!r}")
