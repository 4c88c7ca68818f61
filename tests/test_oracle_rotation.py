"""Pins for oracle.rotation (seeded Haar rotation of the residual).

* SplitMix64 against its published reference outputs (tests/golden);
* the Gaussian draws have mean 0 / variance 1 (statistical, 6 sigma);
* Pi is orthogonal to 1e-13, preserves every row norm and the Frobenius norm
  of a rotated residual to 1e-12 (the invariants a JL rotation must keep);
* Pi is the Q factor with a positive-diagonal R: Pi^T Z is upper triangular
  with a positive diagonal -- independent of LAPACK's sign conventions;
* the same seed regenerates the same Pi, a different seed does not.
"""
import json
import os

import numpy as np
import pytest

from oracle import rotation

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "splitmix64.json")))


def test_splitmix64_reference_vectors():
    v0, v1 = GOLD["vectors"]
    assert rotation.splitmix64(v0["seed"], 3) == [int(x, 16) for x in v0["outputs"]]
    assert rotation.splitmix64(v1["seed"], 3) == v1["outputs_decimal"]


def test_uniforms_open_interval_and_gaussian_moments():
    u = rotation.uniforms(7, 20000)
    assert np.all(u > 0) and np.all(u < 1)
    z = rotation.gaussian_matrix(0x4A4F4C54, 128).ravel()
    n = z.size
    assert abs(z.mean()) < 6 / np.sqrt(n)
    assert abs(z.var() - 1) < 6 * np.sqrt(2 / n)


@pytest.mark.parametrize("d", [64, 128])
def test_orthogonal_and_norm_preserving(d):
    Pi = rotation.rotation(0x4A4F4C54, d)
    assert np.max(np.abs(Pi.T @ Pi - np.eye(d))) < 1e-13
    R = np.random.default_rng(0).standard_normal((500, d)) * 3
    Rp = rotation.rotate(R, Pi)
    assert np.allclose(np.linalg.norm(Rp, axis=1), np.linalg.norm(R, axis=1), rtol=1e-12)
    assert np.linalg.norm(Rp) == pytest.approx(np.linalg.norm(R), rel=1e-12)
    assert np.allclose(rotation.unrotate(Rp, Pi), R, atol=1e-12)


def test_is_q_factor_with_positive_diagonal():
    d = 64
    Z = rotation.gaussian_matrix(11, d)
    Pi = rotation.rotation(11, d)
    R = Pi.T @ Z
    assert np.max(np.abs(np.tril(R, -1))) < 1e-12 * np.max(np.abs(R))
    assert np.all(np.diag(R) > 0)


def test_seed_determinism():
    a = rotation.rotation(5, 64)
    assert np.array_equal(a, rotation.rotation(5, 64))
    assert np.max(np.abs(a - rotation.rotation(6, 64))) > 0.1


def test_array_form_of_the_generator_equals_the_sequential_one():
    from oracle.rotation import splitmix64, splitmix64_array
    for seed in (0, 1, 0x4A4F4C54, (1 << 64) - 1):
        assert splitmix64_array(seed, 257).tolist() == splitmix64(seed, 257)


def test_gaussian_stream_prefix_and_moments():
    from oracle.rotation import gaussian_matrix, gaussians
    z = gaussians(9, 200001)
    assert np.array_equal(gaussian_matrix(9, 16).ravel(), z[:256])
    assert abs(z.mean()) < 5 / np.sqrt(len(z)) and abs(z.var() - 1) < 0.02
