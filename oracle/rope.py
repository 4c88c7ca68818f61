"""Rotary position embedding at float32 angles.

What this module computes: the rotation of a query or key vector to its
token position, with the angle of each feature pair formed in float32 from
the model's float32 inverse frequencies and an integer position.  Sources: the
sarnas.ru JoLT post (section on building cos/sin inside the kernel: float32
angles from int32 positions and the model's inv_freq) and "A JoLT for the KV
cache" (arXiv 2607.12550v4 summary), §3 and §4.5/§5 (keys decomposed before
RoPE, RoPE applied again per decoded tile).

Reading taken: rotate-half pairing (feature i with i + d/2), as in the Llama
family; the angle of pair i at position t is the float32 product
fl32(fl32(t) * inv_freq[i]); cos and sin of that float32 angle are evaluated
in float64:
    y_i       = x_i c_i - x_{i+d/2} s_i
    y_{i+d/2} = x_{i+d/2} c_i + x_i s_i
"""
import numpy as np


def angles(pos, inv_freq):
    """fl32(t * inv_freq) for positions ``pos`` (any shape) -> pos.shape + (d/2,)."""
    p = np.asarray(pos, dtype=np.float32)[..., None]
    f = np.asarray(inv_freq, dtype=np.float32)
    return (p * f).astype(np.float32)


def rope(x, pos, inv_freq):
    """x[..., d] (float64) at positions ``pos`` (broadcast against x[..., 0])."""
    x = np.asarray(x, dtype=np.float64)
    half = x.shape[-1] // 2
    a = angles(pos, inv_freq).astype(np.float64)
    c, s = np.cos(a), np.sin(a)
    lo, hi = x[..., :half], x[..., half:]
    return np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=-1)
