"""Uniform b-bit quantisation of the rotated residual, and code packing.

"A JoLT for the KV cache" (arXiv 2607.12550v4 summary), §3: the rotated
residual is quantised at a selected low bit-width, b = 0 meaning no residual
is stored; the gist.science summaries ("JL-Geroteerd Residu") give
b in {0, 2, 4, 8} and call the quantiser uniform; §1 speaks of packed
residuals.

Readings taken (the pages fix neither granularity, scale nor packing):

* one scale per row, a row being one (layer, head, token) vector of d rotated
  residual entries; symmetric mid-rise grid with L = 2^b - 1 steps:
      delta = fl32(2 max_i |r'_i| / L)
      c_i   = clip(rint(r'_i / delta + L/2), 0, L)     (ties to even)
      deq_i = (c_i - L/2) delta
  and delta = 0 gives c_i = floor(L/2), deq = 0;
* the scale is stored as float32 (4 bytes per row);
* codes are packed least-significant-bits first into bytes, rows of d*b/8
  bytes:  b=2: c0 | c1<<2 | c2<<4 | c3<<6;  b=4: c0 | c1<<4;  b=8: c0.
"""
import numpy as np

BITS = (0, 2, 4, 8)


def levels(bits):
    return (1 << bits) - 1


def quantize_rows(Rp, bits):
    """Rp[..., d] float64 -> (codes uint8 [..., d], delta float32 [...])."""
    L = levels(bits)
    m = np.max(np.abs(Rp), axis=-1)
    delta = (2.0 * m / L).astype(np.float32)
    dd = delta.astype(np.float64)[..., None]
    safe = np.where(dd == 0.0, 1.0, dd)
    c = np.clip(np.rint(Rp / safe + L / 2.0), 0, L)
    c = np.where(dd == 0.0, L // 2, c)
    return c.astype(np.uint8), delta


def dequantize(codes, delta, bits):
    L = levels(bits)
    return (codes.astype(np.float64) - L / 2.0) * delta.astype(np.float64)[..., None]


def pack(codes, bits):
    """codes[..., d] (values < 2^bits) -> bytes[..., d*bits/8], LSB first."""
    per = 8 // bits
    c = codes.astype(np.uint8).reshape(codes.shape[:-1] + (codes.shape[-1] // per, per))
    out = np.zeros(c.shape[:-1], dtype=np.uint8)
    for j in range(per):
        out |= (c[..., j] << np.uint8(j * bits)).astype(np.uint8)
    return out


def unpack(packed, bits, d):
    per = 8 // bits
    mask = np.uint8((1 << bits) - 1)
    out = np.empty(packed.shape + (per,), dtype=np.uint8)
    for j in range(per):
        out[..., j] = (packed >> np.uint8(j * bits)) & mask
    return out.reshape(packed.shape[:-1] + (d,))
