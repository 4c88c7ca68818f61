"""Pins for oracle.allocate (single-multiplier rank/bit allocator).

* m2(d) = E[max_i z_i^2]: closed forms m2(1) = 1 and m2(2) = 1 + 2/pi, and a
  Monte-Carlo estimate at d = 128;
* the chosen allocation fits the budget;
* Lagrangian optimality, by brute force over every joint allocation of two
  tiny cells: no allocation with at most the chosen bytes has a smaller
  total surrogate;
* coordinate-wise search finds the exhaustive argmin on small grids;
* as the budget grows (2, 3, 4, 5x) the total surrogate does not increase,
  the bytes do not decrease, and -- on real compressions of a seeded cache --
  the true relative Frobenius error does not increase;
* b = 0 stores no residual bytes.
"""
import itertools
import math

import numpy as np
import pytest

from oracle import allocate as al
from oracle.compress import budget_for, cell_stats, compress_cell
from oracle.rotation import rotation
from oracle.tucker import reconstruct
from oracle.attention import decode_cell
from workloads import gen


def test_m2_closed_forms():
    assert al.m2(1) == pytest.approx(1.0, abs=1e-10)
    assert al.m2(2) == pytest.approx(1.0 + 2.0 / math.pi, abs=1e-10)


def test_m2_monte_carlo_d128():
    z = np.random.default_rng(0).standard_normal((200000, 128))
    mx = np.max(z * z, axis=1)
    se = mx.std() / math.sqrt(len(mx))
    assert abs(mx.mean() - al.m2(128)) < 5 * se


def small_cells(seed=0, T=64, d=32, gs=1, H=2):
    out = []
    for tau, alpha in ((0, 1.0), (1, 0.3)):
        X = gen.kv_tensor((99, seed, 0, tau), gs, H, T, d, alpha, tau == 0, 2, rank=16)
        out.append(cell_stats(X, 2))
    return out


def all_allocs(st):
    for rT in st.r_T_grid():
        for rF in st.r_F_grid():
            if (rT == 0) != (rF == 0):
                continue
            for b in (0, 2, 4, 8):
                yield int(rT), int(rF), b


@pytest.mark.parametrize("ratio", [2.0, 3.0, 5.0, 8.0])
def test_lagrangian_optimal_by_brute_force(ratio):
    cells = small_cells()
    budget = budget_for(ratio, 1, 2, 32, 64)
    choice, lam = al.allocate(cells, budget)
    nbytes = sum(s.bytes(*c) for s, c in zip(cells, choice))
    D = sum(s.surrogate(*c) for s, c in zip(cells, choice))
    assert nbytes <= budget
    best = math.inf
    for a, b in itertools.product(all_allocs(cells[0]), all_allocs(cells[1])):
        if cells[0].bytes(*a) + cells[1].bytes(*b) <= nbytes:
            best = min(best, cells[0].surrogate(*a) + cells[1].surrogate(*b))
    assert D <= best * (1 + 1e-12)


@pytest.mark.parametrize("lam", [1e-4, 1e-2, 0.1, 1.0, 10.0, 100.0])
def test_coordinate_matches_exhaustive(lam):
    for st in small_cells(1) + small_cells(2, T=128, d=64):
        assert al.choose_coordinate(st, lam) == al.choose_exhaustive(st, lam)


def test_monotone_in_budget_and_true_error():
    T, d, gs, H = 256, 64, 1, 2
    Xs = [gen.kv_tensor((98, 0, 0, tau), gs, H, T, d, a, tau == 0, 2) for tau, a in ((0, 1.0), (1, 0.3))]
    cells = [cell_stats(X, 2) for X in Xs]
    Pi = rotation(3, d)
    prev = None
    for ratio in (5.0, 4.0, 3.0, 2.0):          # growing budget
        choice, lam = al.allocate(cells, budget_for(ratio, 1, H, d, T))
        nbytes = sum(s.bytes(*c) for s, c in zip(cells, choice))
        D = sum(s.surrogate(*c) for s, c in zip(cells, choice))
        err = 0.0
        for X, c in zip(Xs, choice):
            cell = compress_cell(X, *c, "bf16", Pi)
            err += np.sum((decode_cell(cell, 0, d, Pi) - X[0]) ** 2)
        rel = math.sqrt(err / sum(np.sum(X ** 2) for X in Xs))
        if prev is not None:
            assert nbytes >= prev[0] and D <= prev[1] * (1 + 1e-12) and rel <= prev[2] * (1 + 1e-9)
        prev = (nbytes, D, rel)


def test_zero_bits_no_residual_bytes():
    st = small_cells()[0]
    assert st.bytes(32, 16, 0) == 2 * (64 * 32 + 32 * 16 + 2 * 32 * 16)


def test_keys_cheaper_than_values():
    # values (flatter spectrum) receive at least as many bytes as keys
    cells = small_cells(3)
    choice, _ = al.allocate(cells, budget_for(3.0, 1, 2, 32, 64))
    assert cells[1].bytes(*choice[1]) >= cells[0].bytes(*choice[0])


# ------------------------------------------------- discarded-mass tails --
# The surrogate's tails are pinned against the true error of the ST-HOSVD the
# compressor runs (oracle.tucker.st_hosvd, itself pinned by Eckart-Young and
# the ST-HOSVD error identity), never against a restatement of their own
# cumulative sums.
from oracle.tucker import st_hosvd  # noqa: E402


def true_err2(X, rT, rF):
    A, B, G = st_hosvd(X, rT, rF)
    return float(np.sum((X - reconstruct(A, B, G)) ** 2))


def test_tail_T_is_eckart_young_error():
    """One layer, one head, full feature rank: ST-HOSVD is the rank-r_T
    truncated SVD, whose squared error is exactly the discarded token mass."""
    X = gen.kv_tensor((96, 0, 0, 1), 1, 1, 80, 32, 0.3, False, 0, rank=24)
    st = cell_stats(X, 2)
    for r in range(0, 81, 16):
        e = true_err2(X, r, 32) if r else float(np.sum(X ** 2))
        assert float(st.tail_T(r)) == pytest.approx(e, rel=1e-9, abs=1e-9 * st.norm2), r
    # the same through the surrogate at b = 0 (phi = 1)
    for r in (16, 48):
        assert float(st.surrogate(r, 32, 0)) == pytest.approx(true_err2(X, r, 32), rel=1e-9)


def test_tail_F_is_eckart_young_error():
    """Full token rank: ST-HOSVD truncates only the feature mode, and the
    error is exactly the discarded feature mass of the unprojected tensor."""
    X = gen.kv_tensor((96, 1, 0, 0), 2, 2, 40, 32, 1.0, True, 2, rank=12)
    st = cell_stats(X, 2)
    full_T = min(40, 2 * 2 * 32)
    for r in (8, 16, 24):
        assert float(st.tail_F(r)) == pytest.approx(true_err2(X, full_T, r), rel=1e-9)


@pytest.mark.parametrize("seed", range(4))
def test_surrogate_brackets_true_st_hosvd_error(seed):
    """General (r_T, r_F): the true squared error lies between the larger of
    the two tails (each mode alone is an Eckart-Young lower bound) and their
    sum (the ST-HOSVD bound the surrogate prices), and the surrogate at
    b = 0 is never below it."""
    g = np.random.default_rng(seed)
    gs, H, T, d = 2, 3, 64, 32
    X = gen.kv_tensor((95, seed, 0, seed & 1), gs, H, T, d, [1.0, 0.3][seed & 1], True, 2, rank=20)
    st = cell_stats(X, 2)
    for _ in range(6):
        rT = int(g.integers(1, 5)) * 16
        rF = int(g.integers(1, 3)) * 16
        e = true_err2(X, rT, rF)
        lo = max(float(st.tail_T(rT)), float(st.tail_F(rF)))
        hi = float(st.tail_T(rT) + st.tail_F(rF))
        tol = 1e-10 * st.norm2          # rounding of norm2 - cumsum
        assert lo - tol <= e <= hi + tol, (rT, rF, lo, e, hi)
        assert float(st.surrogate(rT, rF, 0)) >= e - tol


def test_tails_fail_on_an_index_shift():
    """An off-by-one in the cumulative-sum index would move every tail by a
    whole squared singular value: the Eckart-Young case tells them apart."""
    X = gen.kv_tensor((96, 2, 0, 1), 1, 1, 64, 32, 0.3, False, 0, rank=24)
    st = cell_stats(X, 2)
    e = true_err2(X, 16, 32)
    assert float(st.tail_T(16)) == pytest.approx(e, rel=1e-9)
    assert abs(float(st.tail_T(16)) - (st.norm2 - np.sum(st.sT2[:15]))) > 1e-3 * e
    assert abs(float(st.tail_T(16)) - (st.norm2 - np.sum(st.sT2[:17]))) > 1e-3 * e
