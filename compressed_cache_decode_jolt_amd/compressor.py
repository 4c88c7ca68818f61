"""GPU compression pipeline (FlashJoLT) over the library's C entry points.

A prefill cache already on the device is compressed group by group:
jolt_flash_spectra gives each cell's allocator inputs, jolt_allocate (host
C++) chooses (r_T, r_F, bits) for every cell under the byte budget, and
jolt_flash_compress_cell builds each stored cell.  The result is the cache
description jolt_load_cache takes.  "A JoLT for the KV cache" (arXiv
2607.12550v4 summary), §3 and §3.1 "Fast variant: FlashJoLT".  Every
arithmetic step runs in the library; this module only sequences the calls.
"""
from . import _jolt as _J


def dense_bytes(n_layers, H, d, T):
    """bf16 K and V bytes of one sequence (the reference the budget divides)."""
    return 2 * n_layers * H * d * T * 2


def compress_cache(groups, H_q, group_start, budget=None, alloc=None, q_cap=256,
                   factor_dtype="bf16", rotation_seed=0x4A4F4C54, oversample=16, power_iters=2,
                   sketch_seed=0, stream=None):
    """groups[g] = (X_K, X_V): device tensors [layers of group g, H, T, d].
    Either ``budget`` (bytes) -- the allocator chooses -- or ``alloc[g] =
    ((r_T, r_F, b) K, (r_T, r_F, b) V)``.  Returns (cache dict, alloc)."""
    XK0 = groups[0][0]
    _, H, T, d = XK0.shape
    fb = 4 if factor_dtype == "f32" else 2
    kw = dict(oversample=oversample, power_iters=power_iters, sketch_seed=sketch_seed,
              stream=stream)
    if alloc is None:
        if budget is None:
            raise ValueError("give a byte budget or an allocation")
        cells = []
        for XK, XV in groups:
            for X in (XK, XV):
                sT2, sF2, n2 = _J.jolt_flash_spectra(X, q_cap, **kw)
                cells.append({"T": T, "d": d, "group_size": X.shape[0], "H": H,
                              "factor_bytes": fb, "sT2": sT2, "sF2": sF2, "norm2": n2,
                              "cap": q_cap})
        choice, _ = _J.jolt_allocate(cells, budget)
        alloc = [(tuple(choice[2 * g]), tuple(choice[2 * g + 1])) for g in range(len(groups))]
    stored = []
    for (XK, XV), (aK, aV) in zip(groups, alloc):
        stored.append(tuple(_J.jolt_flash_compress_cell(X, *a, q_cap, rotation_seed, factor_dtype,
                                                        **kw)
                            for X, a in ((XK, aK), (XV, aV))))
    cache = {"T": T, "H": H, "H_q": H_q, "d": d, "n_layers": group_start[-1],
             "group_start": list(group_start), "factor_dtype": factor_dtype,
             "rotation_seed": int(rotation_seed), "cells": stored}
    return cache, alloc
