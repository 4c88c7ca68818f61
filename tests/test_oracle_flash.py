"""Pins for oracle.flash (FlashJoLT's randomized token-mode SVD).

* exactness: when the token unfolding has rank <= q_cap + oversample, the
  sketch captures its whole column space and the randomized ST-HOSVD equals
  the exact one (tucker.st_hosvd) to rounding, singular values included;
* on data with a spectral gap the leading singular values match numpy's SVD
  closely (Halko-Martinsson-Tropp), and the reconstruction is as good as
  the exact ST-HOSVD's to within a tiny margin;
* the synthetic tail entry is the norm's remainder and the feature spectrum
  is the exact one of the unprojected tensor;
* orth() is the positive-diagonal QR factor; the test matrix is the seeded
  Gaussian stream.
"""
import numpy as np
import pytest

from oracle import flash, tucker
from workloads import gen


def low_rank_X(seed, gs=2, H=2, T=120, d=16, rank=10, noise=0.0):
    g = np.random.default_rng(seed)
    U = g.standard_normal((T, rank))
    X = np.einsum("tr,lhrf->lhtf", U, g.standard_normal((gs, H, rank, d)))
    return X + noise * g.standard_normal(X.shape)


def test_orth_is_positive_diagonal_qr():
    Y = np.random.default_rng(0).standard_normal((50, 7))
    Q = flash.orth(Y)
    assert np.allclose(Q.T @ Q, np.eye(7), atol=1e-13)
    R = Q.T @ Y
    assert np.allclose(np.tril(R, -1), 0, atol=1e-12) and np.all(np.diag(R) > 0)


def test_sketch_matrix_is_the_seeded_stream():
    from oracle.rotation import gaussians
    O = flash.sketch_matrix(5, 30, 7)
    assert O.shape == (30, 7) and np.array_equal(O.ravel(), gaussians(5, 210))


@pytest.mark.parametrize("power_iters", [0, 2])
def test_exact_when_rank_fits_the_sketch(power_iters):
    X = low_rank_X(1, rank=10)
    U, s = flash.randomized_token_basis(X, 10, oversample=4, power_iters=power_iters, sketch_seed=3)
    s_exact = np.linalg.svd(tucker.token_unfolding(X), compute_uv=False)[:10]
    assert np.allclose(s, s_exact, rtol=1e-10)
    for rT, rF in ((10, 16), (6, 8), (3, 5)):
        a = tucker.reconstruct(*flash.flash_st_hosvd(X, rT, rF, 10, 4, power_iters, 3))
        b = tucker.reconstruct(*tucker.st_hosvd(X, rT, rF))
        assert np.max(np.abs(a - b)) <= 1e-9 * np.max(np.abs(b)), (rT, rF)


def test_close_to_exact_with_a_spectral_gap():
    X = gen.kv_tensor((93, 0, 0, 0), 2, 2, 400, 32, 1.0, True, 2, rank=24)
    q = 32
    _, s = flash.randomized_token_basis(X, q, 16, 2, 7)
    s_exact = np.linalg.svd(tucker.token_unfolding(X), compute_uv=False)
    assert np.allclose(s[:24], s_exact[:24], rtol=1e-6)
    for rT, rF in ((16, 16), (24, 32)):
        e_flash = np.sum((X - tucker.reconstruct(*flash.flash_st_hosvd(X, rT, rF, q, 16, 2, 7))) ** 2)
        e_exact = np.sum((X - tucker.reconstruct(*tucker.st_hosvd(X, rT, rF))) ** 2)
        assert e_exact * (1 - 1e-9) <= e_flash <= e_exact * (1 + 1e-4)


def test_spectra_tail_entry_and_feature_spectrum():
    X = low_rank_X(2, rank=12, noise=0.01)
    sT2, sF2, n2 = flash.flash_spectra(X, 8, 4, 2, 1)
    assert len(sT2) == 9
    assert n2 == pytest.approx(float(np.sum(X ** 2)), rel=1e-14)
    assert sT2[-1] == pytest.approx(n2 - np.sum(sT2[:-1]), rel=1e-12, abs=1e-12 * n2)
    e_sT2, e_sF2, _ = tucker.spectra(X)
    assert np.allclose(sF2, e_sF2, rtol=1e-10, atol=1e-10 * n2)
    # the tail entry is the exact discarded token mass (up to the sketch's accuracy)
    assert sT2[-1] == pytest.approx(np.sum(e_sT2[8:]), rel=1e-6)


def test_rank_above_cap_is_refused():
    with pytest.raises(ValueError):
        flash.flash_st_hosvd(low_rank_X(3), 12, 8, 8)
