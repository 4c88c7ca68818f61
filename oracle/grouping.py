"""Alignment-based layer grouping.

TEST INFRASTRUCTURE (see the package docstring).

What this module computes: the partition of a model's layers into groups of
consecutive layers whose token-mode singular vectors align, computed from the
cache being compressed itself.  Source: "A JoLT for the KV cache" (arXiv
2607.12550v4 summary), §3 (consecutive layers grouped by the alignment of
their token-mode singular vectors, no calibration data; 11 groups for
Mistral-7B-v0.3 at T = 1024) and §3.1 (the timing of the fast variant
includes the grouping).

Readings taken where the pages are silent (no alignment measure, threshold
or basis size is printed):

* a layer's token-mode basis U_l is the leading r left singular vectors of
  its token unfolding with keys and values side by side (T x 2 H d), found
  by the same randomized subspace iteration as FlashJoLT (flash.py), seeded;
* the alignment of two layers is ||U_a^T U_b||_F^2 / r, the mean squared
  cosine of their principal angles: 1 for one subspace, about r / T for
  unrelated ones;
* layers l and l + 1 share a group when their alignment is at least tau;
  groups are the maximal runs of such layers, split further so that no group
  has more than max_group layers (0: no limit).
"""
import numpy as np

from .flash import randomized_token_basis


def layer_basis(XK, XV, r, oversample=16, power_iters=2, sketch_seed=0):
    """U (T x r) of one layer: XK, XV [H, T, d] side by side in the token
    unfolding."""
    X = np.concatenate([XK, XV], axis=0)[None]          # [1, 2H, T, d]
    U, _ = randomized_token_basis(X, r, oversample, power_iters, sketch_seed)
    return U


def alignment(Ua, Ub):
    return float(np.sum((Ua.T @ Ub) ** 2) / Ua.shape[1])


def align_groups(layers, r, tau, max_group=0, oversample=16, power_iters=2, sketch_seed=0):
    """layers[l] = (XK, XV), each [H, T, d].  Returns (group_start, a) with
    group_start = [0, ..., n_layers] and a[l] the alignment of l and l + 1."""
    U = [layer_basis(k, v, r, oversample, power_iters, sketch_seed) for k, v in layers]
    a = [alignment(U[l], U[l + 1]) for l in range(len(U) - 1)]
    starts = [0]
    for l in range(1, len(U)):
        size = l - starts[-1]
        if a[l - 1] < tau or (max_group and size >= max_group):
            starts.append(l)
    starts.append(len(U))
    return starts, a
