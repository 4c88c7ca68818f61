"""Seeded generators for synthetic KV caches, queries and compressed caches.

Nothing here is part of the JoLT method: these functions only draw numbers of
the shapes and distributions the decode workloads need.  Both the oracle tests
and the GPU path call them, with the same seeds, so the two sides see the same
inputs.

Raw KV data (one layer group, one of K/V, one sequence)::

    X[l, h] = U diag(s) O[l, h] W^T + 0.05 * N(0, 1)          (T x d)

with U (T x 64) and W (d x 64) i.i.d. N(0, 1) shared by the group's layers and
heads, O[l, h] a Haar-random 64 x 64 orthogonal matrix per (layer, head) so the
head and layer modes stay full rank, and s_i = i^-alpha.  Keys get ``n_out``
seeded outlier channels scaled by 8 after the noise.  This reproduces the
spectral structure the JoLT pages describe: token and feature modes
compressible, head and layer modes not, values harder to compress than keys
(flatter spectrum), keys with fixed outlier channels.
"""
import numpy as np

from .configs import ROTATION_SEED, Config

SEED_ROOT = 0x4A4F4C54
P_U, P_W, P_O, P_NOISE, P_OUT, P_Q, P_SYN = range(7)


def rng(cfg_idx, seq, group, tau, purpose):
    return np.random.default_rng([SEED_ROOT, int(cfg_idx), int(seq), int(group), int(tau),
                                  int(purpose)])


def to_bf16_values(x):
    """Round to the nearest bf16 (ties to even), returned as float32 values."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def _haar(g, n):
    z = g.standard_normal((n, n))
    q, r = np.linalg.qr(z)
    return q * np.where(np.diag(r) >= 0, 1.0, -1.0)


def kv_tensor(key, gs, H, T, d, alpha, is_key, n_out, rank=64, noise=0.05):
    """Synthetic grouped cache X[gs, H, T, d] (float64) for one (seq, group, K/V).

    ``key`` = (cfg_idx, seq, group, tau) selects the seeded streams.
    """
    c, s, g, tau = key
    U = rng(c, s, g, tau, P_U).standard_normal((T, rank))
    W = rng(c, s, g, tau, P_W).standard_normal((d, rank))
    sv = np.arange(1, rank + 1, dtype=np.float64) ** (-alpha)
    go = rng(c, s, g, tau, P_O)
    gn = rng(c, s, g, tau, P_NOISE)
    X = np.empty((gs, H, T, d))
    Us = U * sv
    for l in range(gs):
        for h in range(H):
            O = _haar(go, rank)
            X[l, h] = Us @ (O @ W.T)
            X[l, h] += noise * gn.standard_normal((T, d))
    if is_key and n_out > 0:
        ch = rng(c, s, g, tau, P_OUT).choice(d, size=n_out, replace=False)
        X[..., ch] *= 8.0
    return X


def kv_group(cfg: Config, seq, group, tau, T=None):
    """X for one layer group of a workload: [group_size, H, T, d] float64."""
    T = cfg.T if T is None else T
    return kv_tensor((cfg.idx, seq, group, tau), cfg.group_size, cfg.H, T, cfg.d,
                     cfg.alpha(tau, group), tau == 0, cfg.n_out)


def queries(cfg_idx, seq, layer, H_q, d, q_dtype):
    """q ~ N(0, 1) per (sequence, layer, query head), rounded to the q dtype."""
    q = rng(cfg_idx, seq, layer, 2, P_Q).standard_normal((H_q, d))
    if q_dtype == "bf16":
        return to_bf16_values(q)
    return q.astype(np.float32)


def cfg_queries(cfg: Config, seq, layer):
    return queries(cfg.idx, seq, layer, cfg.H_q, cfg.d, cfg.q_dtype)


def entry_std(alpha, rank=64, noise=0.05):
    sv = np.arange(1, rank + 1, dtype=np.float64) ** (-alpha)
    return float(np.sqrt(np.sum(sv ** 2) + noise ** 2))


def synthetic_cell(g, T, d, gs, H, r_T, r_F, bits, factor_dtype, sigma, resid_frac=0.1):
    """Random stored tensors of one compressed cell (no compressor involved).

    A (T x r_T) and B (d x r_F) have roughly orthonormal columns, G is scaled so
    that A G B^T has entries of std ~``sigma`` with a decaying rank spectrum,
    residual codes are uniform random bytes (a uniform byte is a uniformly
    random group of b-bit codes for b in {2, 4, 8}) and the per-row scales
    correspond to a residual of std ~``resid_frac * sigma``.
    """
    rnd = (lambda x: to_bf16_values(x)) if factor_dtype == "bf16" else \
        (lambda x: np.asarray(x, dtype=np.float32))
    cell = {"r_T": int(r_T), "r_F": int(r_F), "bits": int(bits)}
    A = g.standard_normal((T, r_T)) / np.sqrt(max(T, 1))
    B = g.standard_normal((d, r_F)) / np.sqrt(d)
    w = np.arange(1, r_T + 1, dtype=np.float64) ** -0.5 if r_T > 0 else np.zeros(0)
    if r_T > 0 and r_F > 0:
        w = w * np.sqrt(T * d) * sigma / np.sqrt(np.sum(w ** 2) * r_F)
    G = g.standard_normal((gs, H, r_T, r_F)) * w[None, None, :, None]
    cell["A"], cell["B"], cell["G"] = rnd(A), rnd(B), rnd(G)
    if bits > 0:
        nb = d * bits // 8
        cell["codes"] = g.integers(0, 256, size=(gs, H, T, nb), dtype=np.uint8)
        L = (1 << bits) - 1
        row_max = 3.0 * resid_frac * sigma * (1.0 + 0.25 * np.abs(g.standard_normal((gs, H, T))))
        cell["scales"] = (2.0 * row_max / L).astype(np.float32)
    else:
        cell["codes"] = None
        cell["scales"] = None
    return cell


def synthetic_cache(cfg: Config, alloc, seq=0, T=None, layers=None):
    """A compressed cache with the given allocation and random stored tensors.

    ``alloc[g] = ((r_T, r_F, b) for K, (r_T, r_F, b) for V)``.  ``layers``
    optionally restricts the cache to the first ``layers`` layers (whole
    groups).  Used for timing and for large-shape parity runs where the
    stored values, not the compressor, are what is being decoded.
    """
    T = cfg.T if T is None else T
    n_layers = cfg.n_layers if layers is None else layers
    n_groups = n_layers // cfg.group_size
    cells = []
    for grp in range(n_groups):
        pair = []
        for tau in (0, 1):
            r_T, r_F, b = alloc[grp][tau]
            g = rng(cfg.idx, seq, grp, tau, P_SYN)
            sigma = entry_std(cfg.alpha(tau, grp))
            pair.append(synthetic_cell(g, T, cfg.d, cfg.group_size, cfg.H, r_T, r_F, b,
                                       cfg.factor_dtype, sigma))
        cells.append(pair)
    return {
        "T": T, "H": cfg.H, "H_q": cfg.H_q, "d": cfg.d, "n_layers": n_layers,
        "group_start": [g * cfg.group_size for g in range(n_groups + 1)],
        "factor_dtype": cfg.factor_dtype, "rotation_seed": ROTATION_SEED, "cells": cells,
    }


def rope_inv_freq_input(base, d):
    """The model's RoPE inverse frequencies as the caller hands them in (fp32).

    This is model input data (what a Llama checkpoint stores as ``inv_freq``),
    computed as base^(-2i/d) in float64 and rounded once to float32.
    """
    i = np.arange(d // 2, dtype=np.float64)
    return (float(base) ** (-2.0 * i / d)).astype(np.float32)


def small_cache(seed, T, H, H_q, d, alloc, group_sizes, factor_dtype="bf16",
                sigma=(1.3, 3.4), rotation_seed=ROTATION_SEED):
    """A synthetic compressed cache of arbitrary shape for parity tests.

    ``alloc[g] = ((r_T, r_F, b) K, (r_T, r_F, b) V)``; ``group_sizes[g]`` =
    layers in group g.
    """
    cells = []
    for grp, gs in enumerate(group_sizes):
        pair = []
        for tau in (0, 1):
            r_T, r_F, b = alloc[grp][tau]
            g = rng(1000 + seed, 0, grp, tau, P_SYN)
            pair.append(synthetic_cell(g, T, d, gs, H, r_T, r_F, b, factor_dtype, sigma[tau]))
        cells.append(pair)
    starts = [0]
    for gs in group_sizes:
        starts.append(starts[-1] + gs)
    return {"T": T, "H": H, "H_q": H_q, "d": d, "n_layers": starts[-1], "group_start": starts,
            "factor_dtype": factor_dtype, "rotation_seed": rotation_seed, "cells": cells}
