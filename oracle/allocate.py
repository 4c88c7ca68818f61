"""Joint rank/bit allocation under a global byte budget with one Lagrange
multiplier.

What this module computes: for every cell (layer group, K or V) a triple
(r_T, r_F, b) that minimises the summed estimated squared reconstruction error
of all cells subject to one total byte limit, by pricing bytes with a single
multiplier lambda and bisecting lambda until the limit is met.  Sources: "A
JoLT for the KV cache" (arXiv 2607.12550v4 summary), §3 Method (the
allocator, its error surrogate, the coordinate-wise rank search and the
token-rank cap) and the gist.science summaries, section "Gezamenlijke
Lagrangian Allocatie" (one dual variable; granularity per layer group with
keys and values as separate cells).

Readings taken where the pages are silent:

* cells are (layer group, K or V); candidates r_T in {0, 16, 32, ...} up to
  min(T, |g| H d, cap), r_F in {0, 16, ..., d}, r_T = 0 iff r_F = 0,
  b in {0, 2, 4, 8};
* discarded mass E(r_T, r_F) = min(||X||^2, tail_T(r_T) + tail_F(r_F)) with the
  tails of the squared singular values of the token and feature unfoldings of
  the unprojected tensor (the ST-HOSVD error bound);
* unrecovered fraction phi(0) = 1 and phi(b) = m2(d) / (3 L^2), L = 2^b - 1:
  a uniform quantiser with step delta = 2 max|r'| / L leaves delta^2 / 12 per
  entry, and after a random rotation max_i r'_i^2 ~ (||r||^2 / d) m2(d) with
  m2(d) = E[max_i z_i^2], z ~ N(0, I_d).  m2 is evaluated exactly by
  quadrature of E[Y] = int_0^inf 1 - erf(sqrt(y/2))^d dy;
* surrogate error D = E phi(b); bytes as in accounting.cell_bytes; the
  objective is the absolute summed squared Frobenius error of all cells;
* per cell, for a given lambda: argmin D + lambda * bytes, exhaustive when
  the grid has at most 1e5 points, else coordinate-wise per b (start at
  r_F = max, alternate the argmin over r_T and over r_F until a fixed point,
  at most 20 sweeps); ties go to fewer bytes, then smaller b, smaller r_T,
  smaller r_F;
* lambda: bisection in log space for the smallest lambda whose total bytes
  fit the budget; the feasible end point is returned.
"""
import math
from dataclasses import dataclass
from functools import lru_cache

import numpy as np

from .accounting import cell_bytes
from .quant import BITS, levels

RANK_STEP = 16
EXHAUSTIVE_MAX = 100_000


@lru_cache(maxsize=None)
def m2(d):
    """E[max_i z_i^2] for z ~ N(0, I_d), by quadrature."""
    from scipy import integrate, special

    f = lambda y: 1.0 - special.erf(math.sqrt(y / 2.0)) ** d  # noqa: E731
    val = 0.0
    edges = [0.0, 1.0, 4.0, 16.0, 64.0, 256.0]
    for a, b in zip(edges[:-1], edges[1:]):
        v, _ = integrate.quad(f, a, b, limit=200, epsabs=1e-13, epsrel=1e-13)
        val += v
    return val


def phi(bits, d):
    if bits == 0:
        return 1.0
    L = levels(bits)
    return m2(d) / (3.0 * L * L)


@dataclass
class CellStats:
    T: int
    d: int
    group_size: int
    H: int
    factor_bytes: int
    sT2: np.ndarray   # squared singular values of the token unfolding, descending
    sF2: np.ndarray   # squared singular values of the feature unfolding, descending
    norm2: float
    cap: int = None

    def r_T_grid(self):
        hi = min(self.T, self.group_size * self.H * self.d)
        if self.cap is not None:
            hi = min(hi, self.cap)
        return np.arange(0, hi + 1, RANK_STEP)

    def r_F_grid(self):
        return np.arange(0, self.d + 1, RANK_STEP)

    def tail_T(self, r):
        c = np.concatenate([[0.0], np.cumsum(self.sT2)])
        r = np.minimum(r, len(self.sT2))
        return np.maximum(self.norm2 - c[r], 0.0)

    def tail_F(self, r):
        c = np.concatenate([[0.0], np.cumsum(self.sF2)])
        r = np.minimum(r, len(self.sF2))
        return np.maximum(self.norm2 - c[r], 0.0)

    def surrogate(self, r_T, r_F, bits):
        """D = E(r_T, r_F) phi(b) for a scalar bit-width b."""
        E = np.minimum(self.norm2, self.tail_T(r_T) + self.tail_F(r_F))
        return E * phi(int(bits), self.d)

    def bytes(self, r_T, r_F, bits):
        return cell_bytes(self.T, self.d, self.group_size, self.H, r_T, r_F, bits,
                          self.factor_bytes)


def _pick(obj, nbytes, b, rT, rF):
    """Index of the minimum objective, ties broken by (bytes, b, r_T, r_F)."""
    best = np.min(obj)
    idx = np.nonzero(obj == best)[0]
    if len(idx) == 1:
        return idx[0]
    order = np.lexsort((rF[idx], rT[idx], b[idx], nbytes[idx]))
    return idx[order[0]]


class _Grid:
    """All valid (r_T, r_F, b) candidates of a cell with their D and bytes."""

    def __init__(self, st: CellStats):
        rT, rF = st.r_T_grid(), st.r_F_grid()
        RT, RF, Bb = np.meshgrid(rT, rF, np.array(BITS), indexing="ij")
        RT, RF, Bb = RT.ravel(), RF.ravel(), Bb.ravel()
        ok = (RT == 0) == (RF == 0)
        self.rT, self.rF, self.b = RT[ok], RF[ok], Bb[ok]
        E = np.minimum(st.norm2, st.tail_T(self.rT) + st.tail_F(self.rF))
        ph = np.array([phi(int(x), st.d) for x in BITS])
        self.D = E * ph[np.searchsorted(np.array(BITS), self.b)]
        self.nbytes = st.bytes(self.rT, self.rF, self.b).astype(np.float64)

    def choose(self, lam):
        i = _pick(self.D + lam * self.nbytes, self.nbytes, self.b, self.rT, self.rF)
        return int(self.rT[i]), int(self.rF[i]), int(self.b[i])


def grid_size(st: CellStats):
    nT, nF = len(st.r_T_grid()), len(st.r_F_grid())
    return ((nT - 1) * (nF - 1) + 1) * len(BITS)


def choose_exhaustive(st: CellStats, lam):
    return _Grid(st).choose(lam)


def choose_coordinate(st: CellStats, lam, sweeps=20):
    """Coordinate-wise search over (r_T, r_F) for each b (plus the rank-0
    candidate), then the best over b with the same tie-break."""
    rT_all = st.r_T_grid()[1:]
    rF_all = st.r_F_grid()[1:]
    cands = []
    for b in BITS:
        cands.append((0, 0, b))
        if len(rT_all) == 0 or len(rF_all) == 0:
            continue
        rF = int(rF_all[-1])
        rT = None
        for _ in range(sweeps):
            f = lambda t, s: st.surrogate(t, s, b) + lam * st.bytes(t, s, b)  # noqa: E731
            o = f(rT_all, rF)
            nb = st.bytes(rT_all, rF, b).astype(np.float64)
            i = _pick(o, nb, np.full_like(rT_all, b), rT_all, np.full_like(rT_all, rF))
            new_rT = int(rT_all[i])
            o = f(new_rT, rF_all)
            nb = st.bytes(new_rT, rF_all, b).astype(np.float64)
            j = _pick(o, nb, np.full_like(rF_all, b), np.full_like(rF_all, new_rT), rF_all)
            new_rF = int(rF_all[j])
            if new_rT == rT and new_rF == rF:
                break
            rT, rF = new_rT, new_rF
        cands.append((rT, rF, b))
    c = np.array(cands)
    obj = np.array([st.surrogate(*x) + lam * st.bytes(*x) for x in cands])
    nb = np.array([st.bytes(*x) for x in cands], dtype=np.float64)
    i = _pick(obj, nb, c[:, 2], c[:, 0], c[:, 1])
    return tuple(int(v) for v in c[i])


class Allocator:
    def __init__(self, cells, exhaustive_max=EXHAUSTIVE_MAX):
        self.cells = cells
        self.grids = [(_Grid(st) if grid_size(st) <= exhaustive_max else None) for st in cells]

    def choose_all(self, lam):
        out = []
        for st, g in zip(self.cells, self.grids):
            out.append(g.choose(lam) if g is not None else choose_coordinate(st, lam))
        return out

    def total_bytes(self, choice):
        return sum(st.bytes(*c) for st, c in zip(self.cells, choice))

    def total_surrogate(self, choice):
        return float(sum(st.surrogate(*c) for st, c in zip(self.cells, choice)))

    def solve(self, budget, iters=200):
        """Smallest lambda whose total bytes fit ``budget``: (choice, lambda)."""
        c0 = self.choose_all(0.0)
        if self.total_bytes(c0) <= budget:
            return c0, 0.0
        hi = 1.0
        while self.total_bytes(self.choose_all(hi)) > budget:
            hi *= 2.0
            if hi > 1e300:
                raise ValueError("budget infeasible")
        lo = hi / 2.0
        while self.total_bytes(self.choose_all(lo)) <= budget:
            lo /= 2.0
            if lo < 1e-300:
                return self.choose_all(lo), lo
        for _ in range(iters):
            mid = math.sqrt(lo * hi)
            if not (lo < mid < hi):
                break
            if self.total_bytes(self.choose_all(mid)) <= budget:
                hi = mid
            else:
                lo = mid
        return self.choose_all(hi), hi


def allocate(cells, budget, exhaustive_max=EXHAUSTIVE_MAX):
    """One multiplier for all cells: returns (choices, lambda)."""
    return Allocator(cells, exhaustive_max).solve(budget)
