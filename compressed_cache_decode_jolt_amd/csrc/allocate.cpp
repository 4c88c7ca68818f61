// Joint rank/bit allocation under one byte budget with a single Lagrange
// multiplier (host code; plain C++, no HIP).
//
// "A JoLT for the KV cache" (arXiv 2607.12550v4 summary), §3 Method: per cell
// (layer group, K or V) a token rank, a feature rank and residual bits are
// chosen to minimise the summed estimated reconstruction error subject to a
// global byte budget; the error estimate multiplies the discarded spectral
// mass by the fraction the rotated quantiser leaves unrecovered; the rank
// search is coordinate-wise over the two truncated modes; a token-rank cap
// bounds key rank (§3.1: with FlashJoLT the cap is q_cap).  The gist.science
// summaries, section "Gezamenlijke Lagrangian Allocatie": one dual variable,
// per-group granularity, keys and values separately.
//
// Readings (as the compressor's documentation states them): ranks on a grid
// of 16 with r_T = 0 iff r_F = 0, b in {0, 2, 4, 8}; discarded mass
// min(||X||^2, tail_T(r_T) + tail_F(r_F)) from the two mode spectra;
// unrecovered fraction phi(0) = 1, phi(b) = m2(d) / (3 L^2) with L = 2^b - 1
// and m2(d) = E[max_i z_i^2] for z ~ N(0, I_d); per cell the argmin of
// D + lambda bytes (exhaustive over the grid when it has at most 1e5 points,
// else coordinate-wise per b from r_F = max, at most 20 sweeps), ties to
// fewer bytes, then smaller b, r_T, r_F; lambda by bisection in log space to
// the smallest value whose total bytes fit.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <vector>

#include "errors.h"
#include "jolt.h"

namespace jolt {
}

namespace {

constexpr int kStep = 16;
constexpr int kBits[4] = {0, 2, 4, 8};
constexpr int64_t kExhaustiveMax = 100000;

// m2(d) = E[max_i z_i^2] = int_0^inf 1 - P(z^2 <= y)^d dy
//       = int_0^inf 1 - erf(sqrt(y / 2))^d dy,
// by 32-point Gauss-Legendre on 64 equal panels of each of the intervals
// [0,1], [1,4], [4,16], [16,64], [64,256] (the integrand is below 1e-50
// past 256 for d <= 4096).
double m2(int d) {
  // 32-point Gauss-Legendre nodes on [-1, 1] by Newton iteration on P_32
  static double x[32], w[32];
  static bool init = false;
  if (!init) {
    const int n = 32;
    for (int i = 0; i < n; ++i) {
      double z = std::cos(M_PI * (i + 0.75) / (n + 0.5));
      for (int it = 0; it < 100; ++it) {
        double p0 = 1.0, p1 = z;
        for (int k = 2; k <= n; ++k) {
          const double p2 = ((2.0 * k - 1.0) * z * p1 - (k - 1.0) * p0) / k;
          p0 = p1;
          p1 = p2;
        }
        const double dp = n * (z * p1 - p0) / (z * z - 1.0);
        const double dz = p1 / dp;
        z -= dz;
        if (std::fabs(dz) < 1e-16) {
          x[i] = z;
          w[i] = 2.0 / ((1.0 - z * z) * dp * dp);
          break;
        }
      }
    }
    init = true;
  }
  auto f = [d](double y) { return 1.0 - std::pow(std::erf(std::sqrt(y / 2.0)), (double)d); };
  const double edges[6] = {0.0, 1.0, 4.0, 16.0, 64.0, 256.0};
  double total = 0.0;
  for (int e = 0; e < 5; ++e) {
    const int panels = 64;
    const double h = (edges[e + 1] - edges[e]) / panels;
    for (int p = 0; p < panels; ++p) {
      const double a = edges[e] + p * h, mid = a + h / 2;
      double s = 0.0;
      for (int i = 0; i < 32; ++i) s += w[i] * f(mid + h / 2 * x[i]);
      total += s * h / 2;
    }
  }
  return total;
}

struct Cell {
  int T, d, gs, H, fb, cap;
  std::vector<double> cT, cF;  // [0, cumulative sums of the squared singular values]
  double norm2;
  double phi[4];
  int rT_hi() const {
    int64_t hi = std::min<int64_t>(T, (int64_t)gs * H * d);
    if (cap > 0) hi = std::min<int64_t>(hi, cap);
    return (int)hi;
  }
  double tail(const std::vector<double> &c, int r) const {
    const int i = std::min<int>(r, (int)c.size() - 1);
    return std::max(norm2 - c[i], 0.0);
  }
  double D(int rT, int rF, int bi) const {
    return std::min(norm2, tail(cT, rT) + tail(cF, rF)) * phi[bi];
  }
  int64_t bytes(int rT, int rF, int b) const {
    return (int64_t)fb * ((int64_t)T * rT + (int64_t)d * rF + (int64_t)gs * H * rT * rF) +
           (int64_t)gs * H * T * ((int64_t)d * b / 8 + 4 * (b > 0));
  }
};

struct Choice {
  int rT, rF, bi;
};

// a better than b: smaller objective; ties to fewer bytes, smaller b, r_T, r_F
bool better(double oa, int64_t ba, const Choice &a, double ob, int64_t bb, const Choice &b) {
  if (oa != ob) return oa < ob;
  if (ba != bb) return ba < bb;
  if (kBits[a.bi] != kBits[b.bi]) return kBits[a.bi] < kBits[b.bi];
  if (a.rT != b.rT) return a.rT < b.rT;
  return a.rF < b.rF;
}

Choice choose_exhaustive(const Cell &c, double lam) {
  Choice best{0, 0, 0};
  double bo = 0;
  int64_t bb = 0;
  bool have = false;
  for (int rT = 0; rT <= c.rT_hi(); rT += kStep)
    for (int rF = 0; rF <= c.d; rF += kStep) {
      if ((rT == 0) != (rF == 0)) continue;
      for (int bi = 0; bi < 4; ++bi) {
        const int64_t nb = c.bytes(rT, rF, kBits[bi]);
        const double o = c.D(rT, rF, bi) + lam * (double)nb;
        const Choice ch{rT, rF, bi};
        if (!have || better(o, nb, ch, bo, bb, best)) {
          best = ch, bo = o, bb = nb, have = true;
        }
      }
    }
  return best;
}

Choice choose_coordinate(const Cell &c, double lam) {
  std::vector<int> rTs, rFs;
  for (int r = kStep; r <= c.rT_hi(); r += kStep) rTs.push_back(r);
  for (int r = kStep; r <= c.d; r += kStep) rFs.push_back(r);
  std::vector<Choice> cands;
  for (int bi = 0; bi < 4; ++bi) {
    cands.push_back({0, 0, bi});
    if (rTs.empty() || rFs.empty()) continue;
    const int b = kBits[bi];
    int rF = rFs.back(), rT = -1;
    auto obj = [&](int t, int s) { return c.D(t, s, bi) + lam * (double)c.bytes(t, s, b); };
    for (int sweep = 0; sweep < 20; ++sweep) {
      Choice bt{0, 0, bi};
      double bo = 0;
      int64_t bb = 0;
      bool have = false;
      for (int t : rTs) {
        const Choice ch{t, rF, bi};
        const double o = obj(t, rF);
        const int64_t nb = c.bytes(t, rF, b);
        if (!have || better(o, nb, ch, bo, bb, bt)) bt = ch, bo = o, bb = nb, have = true;
      }
      const int new_rT = bt.rT;
      have = false;
      for (int s : rFs) {
        const Choice ch{new_rT, s, bi};
        const double o = obj(new_rT, s);
        const int64_t nb = c.bytes(new_rT, s, b);
        if (!have || better(o, nb, ch, bo, bb, bt)) bt = ch, bo = o, bb = nb, have = true;
      }
      const int new_rF = bt.rF;
      if (new_rT == rT && new_rF == rF) break;
      rT = new_rT, rF = new_rF;
    }
    cands.push_back({rT, rF, bi});
  }
  Choice best = cands[0];
  double bo = c.D(best.rT, best.rF, best.bi) + lam * (double)c.bytes(best.rT, best.rF, kBits[best.bi]);
  int64_t bb = c.bytes(best.rT, best.rF, kBits[best.bi]);
  for (size_t i = 1; i < cands.size(); ++i) {
    const Choice &ch = cands[i];
    const int64_t nb = c.bytes(ch.rT, ch.rF, kBits[ch.bi]);
    const double o = c.D(ch.rT, ch.rF, ch.bi) + lam * (double)nb;
    if (better(o, nb, ch, bo, bb, best)) best = ch, bo = o, bb = nb;
  }
  return best;
}

int64_t grid_size(const Cell &c) {
  const int64_t nT = c.rT_hi() / kStep + 1, nF = c.d / kStep + 1;
  return ((nT - 1) * (nF - 1) + 1) * 4;
}

}  // namespace

extern "C" jolt_status jolt_allocate(const jolt_alloc_cell *cells, int32_t n_cells, double budget,
                                     int32_t *choice, double *lambda_out) {
  return jolt::guarded("jolt_allocate", [&]() -> jolt_status {
    if (n_cells < 0 || (n_cells > 0 && (!cells || !choice)) || !(budget >= 0.0))
      return jolt::set_error(JOLT_E_INVALID, "jolt_allocate: bad arguments");
    std::vector<Cell> cs(n_cells);
    for (int i = 0; i < n_cells; ++i) {
      const jolt_alloc_cell &in = cells[i];
      if (in.T < 1 || in.d < 1 || in.group_size < 1 || in.n_kv_heads < 1 ||
          (in.factor_bytes != 2 && in.factor_bytes != 4) || in.n_sT2 < 0 || in.n_sF2 < 0 ||
          (in.n_sT2 && !in.sT2) || (in.n_sF2 && !in.sF2) || in.cap < 0 || !(in.norm2 >= 0.0))
        return jolt::set_error(JOLT_E_INVALID, "jolt_allocate: cell %d", i);
      Cell &c = cs[i];
      c.T = in.T, c.d = in.d, c.gs = in.group_size, c.H = in.n_kv_heads, c.fb = in.factor_bytes;
      c.cap = in.cap;
      c.norm2 = in.norm2;
      c.cT.assign(1, 0.0);
      for (int k = 0; k < in.n_sT2; ++k) c.cT.push_back(c.cT.back() + in.sT2[k]);
      c.cF.assign(1, 0.0);
      for (int k = 0; k < in.n_sF2; ++k) c.cF.push_back(c.cF.back() + in.sF2[k]);
      c.phi[0] = 1.0;
      const double m = m2(c.d);
      for (int bi = 1; bi < 4; ++bi) {
        const double L = (double)((1 << kBits[bi]) - 1);
        c.phi[bi] = m / (3.0 * L * L);
      }
    }
    std::vector<char> exh(n_cells);
    for (int i = 0; i < n_cells; ++i) exh[i] = grid_size(cs[i]) <= kExhaustiveMax;
    std::vector<Choice> cur(n_cells);
    auto choose_all = [&](double lam) {
      int64_t total = 0;
      for (int i = 0; i < n_cells; ++i) {
        cur[i] = exh[i] ? choose_exhaustive(cs[i], lam) : choose_coordinate(cs[i], lam);
        total += cs[i].bytes(cur[i].rT, cur[i].rF, kBits[cur[i].bi]);
      }
      return total;
    };
    double lam = 0.0;
    if ((double)choose_all(0.0) > budget) {
      double hi = 1.0;
      while ((double)choose_all(hi) > budget) {
        hi *= 2.0;
        if (hi > 1e300) return jolt::set_error(JOLT_E_INVALID, "jolt_allocate: budget infeasible");
      }
      double lo = hi / 2.0;
      bool done = false;
      while ((double)choose_all(lo) <= budget) {
        lo /= 2.0;
        if (lo < 1e-300) {
          lam = lo;
          done = true;
          break;
        }
      }
      if (!done) {
        for (int it = 0; it < 200; ++it) {
          const double mid = std::sqrt(lo * hi);
          if (!(lo < mid && mid < hi)) break;
          if ((double)choose_all(mid) <= budget)
            hi = mid;
          else
            lo = mid;
        }
        lam = hi;
      }
      choose_all(lam);
    }
    for (int i = 0; i < n_cells; ++i) {
      choice[3 * i] = cur[i].rT;
      choice[3 * i + 1] = cur[i].rF;
      choice[3 * i + 2] = kBits[cur[i].bi];
    }
    if (lambda_out) *lambda_out = lam;
    return jolt::set_error(JOLT_OK, "");
  });
}
