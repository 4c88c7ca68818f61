"""Pins for oracle.quant (uniform b-bit residual quantiser and packing).

* every entry within delta/2 of its dequantised value, codes in [0, L];
* brute force: each code is the nearest of all 2^b grid points;
* values already on the grid quantise exactly;
* delta = 0 rows decode to 0;
* pack -> unpack is the identity; hand-packed bytes for b = 2, 4, 8;
* with a random rotation, the unrecovered energy fraction on Gaussian rows
  matches the allocator's phi(b) model (this fails if the step were max/L
  instead of 2 max/L, or the grid mis-centred).
"""
import numpy as np
import pytest

from oracle import quant
from oracle.allocate import phi


@pytest.mark.parametrize("b", [2, 4, 8])
def test_error_bound_and_range(b):
    x = np.random.default_rng(b).standard_normal((300, 64)) * np.exp(np.random.default_rng(9).standard_normal((300, 1)))
    c, delta = quant.quantize_rows(x, b)
    L = quant.levels(b)
    assert c.max() <= L
    deq = quant.dequantize(c, delta, b)
    assert np.all(np.abs(x - deq) <= delta.astype(np.float64)[:, None] / 2 * (1 + 1e-12))


@pytest.mark.parametrize("b", [2, 4])
def test_brute_force_nearest(b):
    x = np.random.default_rng(3).standard_normal((50, 16))
    c, delta = quant.quantize_rows(x, b)
    L = quant.levels(b)
    grid = (np.arange(L + 1) - L / 2)[None, None, :] * delta.astype(np.float64)[:, None, None]
    dist = np.abs(x[:, :, None] - grid)
    assert np.all(dist[np.arange(50)[:, None], np.arange(16)[None, :], c.astype(int)]
                  <= dist.min(axis=-1) + 1e-15)


def test_grid_points_exact():
    b, L = 8, 255
    delta = np.float32(0.0625)
    c = np.random.default_rng(4).integers(0, L + 1, size=(20, 32))
    c[:, 0] = L          # make the max |value| exactly L/2 * delta
    x = (c - L / 2) * np.float64(delta)
    cq, dq = quant.quantize_rows(x, b)
    assert dq[0] == delta
    assert np.array_equal(cq, c)


def test_zero_row():
    c, delta = quant.quantize_rows(np.zeros((2, 8)), 4)
    assert np.all(delta == 0) and np.all(c == 7)
    assert np.all(quant.dequantize(c, delta, 4) == 0)


def test_pack_hand_examples():
    assert quant.pack(np.array([[1, 2, 3, 0]]), 2).tolist() == [[1 | 2 << 2 | 3 << 4]]
    assert quant.pack(np.array([[0xA, 0x5, 0xF, 0x0]]), 4).tolist() == [[0x5A, 0x0F]]
    assert quant.pack(np.array([[7, 200]]), 8).tolist() == [[7, 200]]


@pytest.mark.parametrize("b", [2, 4, 8])
def test_pack_roundtrip(b):
    c = np.random.default_rng(b).integers(0, 1 << b, size=(3, 5, 128)).astype(np.uint8)
    p = quant.pack(c, b)
    assert p.shape == (3, 5, 128 * b // 8)
    assert np.array_equal(quant.unpack(p, b, 128), c)


@pytest.mark.parametrize("b", [2, 4, 8])
def test_unrecovered_fraction_matches_phi(b):
    from oracle.rotation import rotation
    d = 128
    Pi = rotation(1, d)
    r = np.random.default_rng(5).standard_normal((20000, d))
    rp = r @ Pi
    c, delta = quant.quantize_rows(rp, b)
    err = np.sum((rp - quant.dequantize(c, delta, b)) ** 2) / np.sum(r ** 2)
    assert err == pytest.approx(phi(b, d), rel=0.03)
