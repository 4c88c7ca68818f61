"""Rounding of the stored factors to their storage dtype.

The JoLT summary's reproducibility statement ("A JoLT for the KV cache",
arXiv 2607.12550v4, Reproducibility Statement) runs the models in bf16 and the
decomposition numerics in float32.  Reading taken here: the factors A, B and G
are computed in float64, then stored in the cache's factor dtype (bf16, or
fp32 for the all-fp32 workload) with round-to-nearest-even.  bf16 rounding is
float64 -> float32 (RNE) -> bf16 (RNE on the upper 16 bits of the float32).
"""
import numpy as np


def round_f32(x):
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def round_bf16(x):
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    u = (u + np.uint64(0x7FFF) + lsb) & np.uint64(0xFFFF0000)
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def round_to(x, dtype):
    """Round to the storage dtype; "f64" (tests only) keeps the value."""
    if dtype == "f64":
        return np.asarray(x, dtype=np.float64)
    if dtype == "f32":
        return round_f32(x)
    if dtype == "bf16":
        return round_bf16(x)
    raise ValueError(dtype)
