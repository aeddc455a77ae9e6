"""bf16 decoding for the oracle.

A bf16 value is the upper half of an IEEE binary32: its 16 bits, shifted left
by 16, are the float32 with the same value.  Every bf16 is therefore exact in
float32 and in float64.
"""

import numpy as np


def bf16_to_f32(u16: np.ndarray) -> np.ndarray:
    return (np.asarray(u16, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_to_f64(u16: np.ndarray) -> np.ndarray:
    with np.errstate(invalid="ignore"):  # NaN bit patterns stay NaN
        return bf16_to_f32(u16).astype(np.float64)
