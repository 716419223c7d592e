"""Storage-type helpers of the oracle (its own copy; shares nothing with the
library).  bf16 is carried as uint16 bit patterns: the top half of an IEEE
f32, rounded to nearest with ties to even."""
import numpy as np


def bf16_to_f64(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def round_bf16(x) -> np.ndarray:
    """Round to the nearest bf16 value (ties to even) via f32, returning the
    value as f64.  Used where the library stores an intermediate in bf16 that
    a later step reads back (e.g. the saved softmax output)."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    out = r.astype(np.uint32).view(np.float32).astype(np.float64)
    return np.where(np.isnan(f), np.nan, out)


def round_f32(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def to_f64(a, dtype: str = "f32") -> np.ndarray:
    """Widen a stored tensor to f64: f32/f64 arrays directly, bf16 bit
    patterns exactly."""
    if dtype == "bf16":
        return bf16_to_f64(a)
    return np.asarray(a, dtype=np.float64)
