"""Partial Tucker decomposition of a grouped KV cache by ST-HOSVD.

What this module computes: for one cell, the layer-group cache viewed as a
4-way array (layers, heads, tokens, features), an orthonormal token basis A
and feature basis B common to every layer and head of the group, and a core
G[l, h] per layer and head, by sequentially truncated HOSVD -- the token mode
first, then the feature mode of the token-projected array; the layer and head
modes are left untruncated.  Sources: "A JoLT for the KV cache" (arXiv
2607.12550v4 summary), §3 Method; the gist.science summaries, section
"Partiële Tucker Decompositie" / "Décomposition de Tucker Partielle".

Tensor layout: X[l, h, t, f] with shape (|g|, H, T, d).

* token unfolding   M_T(X) in R^{T x |g| H d}, columns ordered (l, h, f);
* feature unfolding M_F(Y) in R^{d x |g| H r}, columns ordered (l, h, t).

ST-HOSVD(X, r_T, r_F):
  1. A = leading r_T left singular vectors of M_T(X)            (T x r_T)
  2. Y[l, h] = A^T X[l, h]                                        (r_T x d)
  3. B = leading r_F left singular vectors of M_F(Y)            (d x r_F)
  4. G[l, h] = Y[l, h] B                                          (r_T x r_F)
and the reconstruction is X~[l, h] = A G[l, h] B^T.
"""
import numpy as np


def token_unfolding(X):
    gs, H, T, d = X.shape
    return np.transpose(X, (2, 0, 1, 3)).reshape(T, gs * H * d)


def feature_unfolding(Y):
    gs, H, r, d = Y.shape
    return np.transpose(Y, (3, 0, 1, 2)).reshape(d, gs * H * r)


def left_singular(M, r, method="auto"):
    """Leading r left singular vectors of M and all its singular values.

    ``method="svd"`` uses ``numpy.linalg.svd``; ``"gram"`` diagonalises the
    smaller Gram matrix with ``numpy.linalg.eigh`` (U = M V / sigma when the
    Gram matrix is M^T M).  ``"auto"`` picks svd for small matrices.
    Singular vectors are unique only up to sign; only the subspace matters.
    """
    m, n = M.shape
    if method == "auto":
        method = "svd" if m * n <= 4_000_000 else "gram"
    if method == "svd":
        U, s, _ = np.linalg.svd(M, full_matrices=False)
        return U[:, :r], s
    if m <= n:
        w, V = np.linalg.eigh(M @ M.T)
        order = np.argsort(w)[::-1]
        w, V = np.clip(w[order], 0.0, None), V[:, order]
        return V[:, :r], np.sqrt(w)
    w, V = np.linalg.eigh(M.T @ M)
    order = np.argsort(w)[::-1]
    w, V = np.clip(w[order], 0.0, None), V[:, order]
    s = np.sqrt(w)
    Vr = V[:, :r]
    U = (M @ Vr) / s[:r]
    # re-orthonormalise (keeps the span; removes Gram-route rounding drift)
    U, _ = np.linalg.qr(U)
    s_full = np.zeros(min(m, n))
    s_full[: len(s)] = s[: min(m, n)]
    return U, s_full


def singular_values(M):
    """All singular values of M via the smaller Gram matrix."""
    m, n = M.shape
    Gm = M @ M.T if m <= n else M.T @ M
    w = np.linalg.eigvalsh(Gm)[::-1]
    return np.sqrt(np.clip(w, 0.0, None))


def st_hosvd(X, r_T, r_F, method="auto"):
    """Returns (A, B, G) with A (T x r_T), B (d x r_F), G (|g|, H, r_T, r_F)."""
    gs, H, T, d = X.shape
    if r_T == 0 or r_F == 0:
        return np.zeros((T, 0)), np.zeros((d, 0)), np.zeros((gs, H, 0, 0))
    A, _ = left_singular(token_unfolding(X), r_T, method)
    Y = np.einsum("tr,lhtf->lhrf", A, X, optimize=True)
    B, _ = left_singular(feature_unfolding(Y), r_F, method)
    G = Y @ B
    return A, B, G


def reconstruct(A, B, G):
    """X~[l, h] = A G[l, h] B^T, shape (|g|, H, T, d)."""
    gs, H = G.shape[:2]
    T, d = A.shape[0], B.shape[0]
    if A.shape[1] == 0:
        return np.zeros((gs, H, T, d))
    return np.einsum("tr,lhrs,fs->lhtf", A, G, B, optimize=True)


def spectra(X):
    """Allocator inputs from the unprojected tensor: squared singular values
    of the token and feature unfoldings (descending) and ||X||_F^2."""
    sT = singular_values(token_unfolding(X))
    sF = singular_values(np.transpose(X, (3, 0, 1, 2)).reshape(X.shape[3], -1))
    return sT ** 2, sF ** 2, float(np.sum(X * X))
