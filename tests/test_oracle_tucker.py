"""Pins for oracle.tucker (ST-HOSVD on the token and feature modes).

* full token and feature ranks reproduce X to 1e-12 (closed form: both
  projections are the identity on the data's span);
* one layer, one head, full feature rank: the token truncation is the
  Eckart-Young truncated SVD from numpy.linalg.svd (textbook routine);
* the ST-HOSVD error identity ||X - X~||^2 = sum_{i>r_T} sigma_T,i(X)^2 +
  sum_{j>r_F} sigma_F,j(Y)^2 with Y the token-projected tensor
  (Vannieuwenhoven, Vandebril, Meerbergen 2012) -- this also fails if the
  feature basis were taken from the unprojected tensor or the order swapped;
* A and B have orthonormal columns; the svd and Gram routes agree.
"""
import numpy as np
import pytest

from oracle import tucker


def rand_X(seed, gs=2, H=3, T=40, d=16, rank=None):
    g = np.random.default_rng(seed)
    X = g.standard_normal((gs, H, T, d))
    if rank:
        U = g.standard_normal((T, rank))
        X = np.einsum("tr,lhrf->lhtf", U, g.standard_normal((gs, H, rank, d))) + 1e-3 * X
    return X


@pytest.mark.parametrize("method", ["svd", "gram"])
@pytest.mark.parametrize("shape", [(2, 3, 40, 16), (1, 2, 200, 8), (3, 1, 10, 32)])
def test_full_rank_exact(shape, method):
    X = rand_X(0, *shape)
    gs, H, T, d = shape
    A, B, G = tucker.st_hosvd(X, min(T, gs * H * d), d, method)
    Xt = tucker.reconstruct(A, B, G)
    assert np.linalg.norm(X - Xt) / np.linalg.norm(X) <= 1e-12


def test_eckart_young_single_slice():
    X = rand_X(1, 1, 1, 50, 12)
    for r in (1, 3, 7):
        A, B, G = tucker.st_hosvd(X, r, 12)
        U, s, Vt = np.linalg.svd(X[0, 0], full_matrices=False)
        ey = (U[:, :r] * s[:r]) @ Vt[:r]
        assert np.allclose(tucker.reconstruct(A, B, G)[0, 0], ey, atol=1e-12)


@pytest.mark.parametrize("rT,rF", [(5, 3), (12, 8), (30, 16), (1, 1)])
def test_error_identity(rT, rF):
    X = rand_X(2, rank=20)
    A, B, G = tucker.st_hosvd(X, rT, rF)
    err2 = np.sum((X - tucker.reconstruct(A, B, G)) ** 2)
    sT = np.linalg.svd(tucker.token_unfolding(X), compute_uv=False)
    Y = np.einsum("tr,lhtf->lhrf", A, X)
    sF = np.linalg.svd(tucker.feature_unfolding(Y), compute_uv=False)
    want = np.sum(sT[rT:] ** 2) + np.sum(sF[rF:] ** 2)
    assert err2 == pytest.approx(want, rel=1e-9, abs=1e-9)


def test_orthonormal_factors_and_shared_bases():
    X = rand_X(3)
    A, B, G = tucker.st_hosvd(X, 9, 6)
    assert np.allclose(A.T @ A, np.eye(9), atol=1e-12)
    assert np.allclose(B.T @ B, np.eye(6), atol=1e-12)
    assert G.shape == (2, 3, 9, 6)     # core keeps layer and head modes at full size


def test_svd_and_gram_routes_agree():
    X = rand_X(4, 2, 2, 300, 16, rank=12)   # T > |g| H d: the Gram route works on M^T M
    for rT, rF in ((10, 8), (40, 16)):
        a = tucker.reconstruct(*tucker.st_hosvd(X, rT, rF, "svd"))
        b = tucker.reconstruct(*tucker.st_hosvd(X, rT, rF, "gram"))
        assert np.max(np.abs(a - b)) <= 1e-10 * np.max(np.abs(a))


def test_spectra_match_svd():
    X = rand_X(5)
    sT2, sF2, n2 = tucker.spectra(X)
    assert np.allclose(sT2[:16], np.linalg.svd(tucker.token_unfolding(X), compute_uv=False)[:16] ** 2)
    MF = np.transpose(X, (3, 0, 1, 2)).reshape(16, -1)
    assert np.allclose(sF2, np.linalg.svd(MF, compute_uv=False) ** 2)
    assert n2 == pytest.approx(np.sum(sT2)) and n2 == pytest.approx(np.sum(sF2))


def test_zero_rank_is_empty():
    X = rand_X(6)
    A, B, G = tucker.st_hosvd(X, 0, 0)
    assert np.all(tucker.reconstruct(A, B, G) == 0)
