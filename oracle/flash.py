"""FlashJoLT: the compressor with a randomized token-mode SVD.

TEST INFRASTRUCTURE (see the package docstring).

What this module computes.  "A JoLT for the KV cache" (arXiv 2607.12550v4
summary), §3.1 "Fast variant: FlashJoLT" and App. A, and the gist.science
summaries (section "FlashJoLT (Snelle Variant)"): the exact token-mode SVD of
ST-HOSVD is replaced by a randomized low-rank SVD that finds only the leading
q_cap token-mode directions; the feature mode keeps its exact SVD and the
allocator is unchanged; the energy of the spectrum that was not computed is
estimated from the tensor's norm and appended as one synthetic tail entry,
and q_cap also caps the token rank the allocator may buy.

Readings taken where the pages are silent (they name no algorithm variant,
oversampling, power iterations or random distribution):

* the randomized SVD is randomized subspace iteration (Halko, Martinsson and
  Tropp 2011, "Finding structure with randomness", Algorithms 4.4 and 5.1):
  a Gaussian test matrix Omega (N x k, k = q_cap + oversample), Y = M Omega,
  Q = orth(Y); then `power_iters` times: Q = orth(M orth(M^T Q)); finally
  the small matrix Q^T M is decomposed and its left singular vectors are
  mapped back through Q;
* orth(.) is the QR factor with a positive diagonal in R (unique for a full
  column rank input);
* Omega's entries are standard normals from SplitMix64 (the generator of the
  rotation, see rotation.py), seeded with `sketch_seed`, filling Omega row by
  row;
* the synthetic tail entry is max(||X||^2 - sum of the q_cap squared
  singular values, 0).
"""
import numpy as np

from .rotation import gaussians
from .tucker import feature_unfolding, token_unfolding


def orth(Y):
    """Q of the QR factorisation of Y with R's diagonal made positive."""
    Q, R = np.linalg.qr(Y)
    return Q * np.where(np.diag(R) >= 0.0, 1.0, -1.0)


def sketch_matrix(seed, n_rows, k):
    """The Gaussian test matrix Omega (n_rows x k), row-major from the seed."""
    return gaussians(seed, n_rows * k).reshape(n_rows, k)


def randomized_token_basis(X, q_cap, oversample=16, power_iters=2, sketch_seed=0):
    """Leading q_cap left singular vectors (T x q_cap) and singular values of
    the token unfolding of X, by randomized subspace iteration."""
    M = token_unfolding(X)                       # T x N
    T, N = M.shape
    k = min(q_cap + oversample, T, N)
    Omega = sketch_matrix(sketch_seed, N, k)
    Q = orth(M @ Omega)
    for _ in range(power_iters):
        Q = orth(M @ orth(M.T @ Q))
    Bs = Q.T @ M                                 # k x N
    Ub, s, _ = np.linalg.svd(Bs, full_matrices=False)
    q = min(q_cap, k)
    return Q @ Ub[:, :q], s[:q]


def flash_spectra(X, q_cap, oversample=16, power_iters=2, sketch_seed=0):
    """Allocator inputs of FlashJoLT: the q_cap leading squared token-mode
    singular values followed by the synthetic tail entry, the exact squared
    feature-mode singular values of the unprojected tensor, and ||X||^2."""
    _, s = randomized_token_basis(X, q_cap, oversample, power_iters, sketch_seed)
    norm2 = float(np.sum(X * X))
    sT2 = s ** 2
    tail = max(norm2 - float(np.sum(sT2)), 0.0)
    MF = np.transpose(X, (3, 0, 1, 2)).reshape(X.shape[3], -1)
    sF2 = np.sort(np.clip(np.linalg.eigvalsh(MF @ MF.T), 0.0, None))[::-1]
    return np.concatenate([sT2, [tail]]), sF2, norm2


def flash_st_hosvd(X, r_T, r_F, q_cap, oversample=16, power_iters=2, sketch_seed=0):
    """ST-HOSVD with the randomized token basis (r_T <= q_cap): returns
    (A, B, G) as tucker.st_hosvd does."""
    gs, H, T, d = X.shape
    if r_T == 0 or r_F == 0:
        return np.zeros((T, 0)), np.zeros((d, 0)), np.zeros((gs, H, 0, 0))
    if r_T > q_cap:
        raise ValueError("r_T above the token-rank cap")
    U, _ = randomized_token_basis(X, q_cap, oversample, power_iters, sketch_seed)
    A = U[:, :r_T]
    Y = np.einsum("tr,lhtf->lhrf", A, X, optimize=True)
    MF = feature_unfolding(Y)
    w, V = np.linalg.eigh(MF @ MF.T)
    B = V[:, np.argsort(w)[::-1][:r_F]]
    G = Y @ B
    return A, B, G


def flash_compress_cell(X, r_T, r_F, bits, factor_dtype, Pi, q_cap, oversample=16, power_iters=2,
                        sketch_seed=0):
    """One stored cell as oracle.compress.compress_cell builds it, with the
    FlashJoLT token basis in place of the exact one."""
    from .compress import residual_cell
    A, B, G = flash_st_hosvd(X, r_T, r_F, q_cap, oversample, power_iters, sketch_seed)
    return residual_cell(X, A, B, G, r_T, r_F, bits, factor_dtype, Pi)


def flash_compress(groups, budget, factor_dtype, rotation_seed, H_q, group_start, q_cap,
                   oversample=16, power_iters=2, sketch_seed=0):
    """The FlashJoLT pipeline: spectra of every cell (q_cap token energies,
    synthetic tail entry, exact feature energies), the allocator under the
    byte budget with token ranks capped at q_cap, then each cell compressed.
    Returns (cache, allocation)."""
    from .allocate import CellStats, allocate
    from .compress import compress
    fb = 4 if factor_dtype == "f32" else 2
    stats = []
    for XK, XV in groups:
        for X in (XK, XV):
            gs, H, T, d = X.shape
            sT2, sF2, n2 = flash_spectra(X, q_cap, oversample, power_iters, sketch_seed)
            stats.append(CellStats(T=T, d=d, group_size=gs, H=H, factor_bytes=fb, sT2=sT2,
                                   sF2=sF2, norm2=n2, cap=q_cap))
    choice, _ = allocate(stats, budget)
    alloc = [(tuple(choice[2 * g]), tuple(choice[2 * g + 1])) for g in range(len(groups))]
    from .rotation import rotation
    Pi = rotation(rotation_seed, groups[0][0].shape[3])
    cells = [tuple(flash_compress_cell(X, *a, factor_dtype, Pi, q_cap, oversample, power_iters,
                                       sketch_seed) for X, a in ((XK, aK), (XV, aV)))
             for (XK, XV), (aK, aV) in zip(groups, alloc)]
    XK0 = groups[0][0]
    cache = {"T": XK0.shape[2], "H": XK0.shape[1], "H_q": H_q, "d": XK0.shape[3],
             "n_layers": group_start[-1], "group_start": list(group_start),
             "factor_dtype": factor_dtype, "rotation_seed": int(rotation_seed), "cells": cells}
    return cache, alloc
