"""Exact bf16 -> float64 upcast (test infrastructure; see package docstring).

A bf16 value is the upper 16 bits of an IEEE-754 binary32 value. Shifting the
16-bit pattern left by 16 gives that binary32 value exactly, and binary32 ->
binary64 widening is exact, so the upcast loses nothing (NaN and Inf included).
numpy has no bf16 type, so bf16 tensors travel as uint16 bit patterns.
"""
import numpy as np


def bf16_bits_to_f64(bits) -> np.ndarray:
    """uint16 (or int16) bf16 bit patterns, any shape -> float64, exactly."""
    a = np.asarray(bits)
    if a.dtype == np.int16:
        a = a.view(np.uint16)
    if a.dtype != np.uint16:
        raise TypeError(f"expected uint16 bf16 bit patterns, got {a.dtype}")
    f32 = (a.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return f32.astype(np.float64)
