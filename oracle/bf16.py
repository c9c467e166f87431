"""Exact bfloat16 decoding (test infrastructure, see the package docstring).

A bfloat16 value is the upper 16 bits of an IEEE float32, so shifting the
bits left by 16 gives the float32 exactly, and float32 -> float64 is exact.
"""
import numpy as np


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """uint16 bfloat16 bit patterns -> float64 (exact)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def to_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Decode a stored tensor ("bf16" bits or "f32") to float64."""
    if dtype == "bf16":
        return bf16_to_f64(x)
    return np.asarray(x, dtype=np.float32).astype(np.float64)
