"""The JoLT compressor: grouped prefill cache -> stored cells.

What this module computes: for each cell, the ST-HOSVD factors
(tucker.st_hosvd) rounded to the storage dtype, the residual X - X~ of that
stored reconstruction rotated by Pi (rotation) and quantised to b bits with
its codes packed (quant); the ranks and bits come from the single-multiplier
allocator (allocate).  Sources: "A JoLT for the KV cache" (arXiv
2607.12550v4 summary), Abstract and §3; the gist.science summaries, section
"JL-Geroteerd Residu" (R = X - X~).

Reading taken: X~ is the reconstruction from the *stored* (dtype-rounded)
factors, so the residual also absorbs factor rounding -- the decoder adds the
residual to exactly what it reconstructs.

A compressed cache is a plain dict:
  T, H, H_q, d, n_layers, group_start, factor_dtype, rotation_seed,
  cells[g] = (K cell, V cell), each cell a dict with r_T, r_F, bits,
  A [T, r_T], B [d, r_F], G [|g|, H, r_T, r_F] (float32 arrays holding values
  of the factor dtype), codes uint8 [|g|, H, T, d*bits/8] and scales float32
  [|g|, H, T] (None when bits == 0).
"""
import numpy as np

from . import allocate as alloc_mod
from .accounting import dense_kv_bytes
from .quant import pack, quantize_rows
from .rotation import rotate, rotation
from .storage import round_to
from .tucker import reconstruct, spectra, st_hosvd


def compress_cell(X, r_T, r_F, bits, factor_dtype, Pi):
    A, B, G = st_hosvd(X, r_T, r_F)
    return residual_cell(X, A, B, G, r_T, r_F, bits, factor_dtype, Pi)


def residual_cell(X, A, B, G, r_T, r_F, bits, factor_dtype, Pi):
    """Stored cell from exact factors: rounded to the storage dtype, then the
    residual against that stored reconstruction rotated, quantised, packed."""
    A, B, G = round_to(A, factor_dtype), round_to(B, factor_dtype), round_to(G, factor_dtype)
    keep = np.float64 if factor_dtype == "f64" else np.float32
    cell = {"r_T": int(r_T), "r_F": int(r_F), "bits": int(bits),
            "A": A.astype(keep), "B": B.astype(keep), "G": G.astype(keep),
            "codes": None, "scales": None}
    if bits > 0:
        R = X - reconstruct(A, B, G)
        codes, delta = quantize_rows(rotate(R, Pi), bits)
        cell["codes"] = pack(codes, bits)
        cell["scales"] = delta
    return cell


def cell_stats(X, factor_bytes, cap=None):
    gs, H, T, d = X.shape
    sT2, sF2, n2 = spectra(X)
    return alloc_mod.CellStats(T=T, d=d, group_size=gs, H=H, factor_bytes=factor_bytes,
                               sT2=sT2, sF2=sF2, norm2=n2, cap=cap)


def budget_for(ratio, n_layers, H, d, T):
    """Byte budget = dense bf16 KV bytes of one sequence / compression ratio."""
    return dense_kv_bytes(n_layers, H, d, T, 2) / ratio


def compress(groups, alloc, factor_dtype, rotation_seed, H_q, group_start):
    """groups[g] = (X_K, X_V) each [|g|, H, T, d]; alloc[g] = ((r_T, r_F, b) K, (...) V)."""
    XK0 = groups[0][0]
    _, H, T, d = XK0.shape
    Pi = rotation(rotation_seed, d)
    cells = []
    for (XK, XV), (aK, aV) in zip(groups, alloc):
        cells.append((compress_cell(XK, *aK, factor_dtype, Pi),
                      compress_cell(XV, *aV, factor_dtype, Pi)))
    return {"T": T, "H": H, "H_q": H_q, "d": d, "n_layers": group_start[-1],
            "group_start": list(group_start), "factor_dtype": factor_dtype,
            "rotation_seed": int(rotation_seed), "cells": cells}
