"""Exact widening of stored inputs to float64 (oracle; test infrastructure only).

bfloat16 values are the top 16 bits of an IEEE float32, so shifting the stored bits
left by 16 gives the float32 with the same value, which float64 holds exactly.
"""
import numpy as np


def widen(x: np.ndarray) -> np.ndarray:
    """uint16 bfloat16 bit patterns or float32 values -> float64 with identical values."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if x.dtype == np.float32 or x.dtype == np.float64:
        return x.astype(np.float64)
    raise TypeError(f"unsupported stored dtype {x.dtype}")
