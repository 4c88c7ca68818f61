// Regeneration of the residual rotation Pi from its seed.
//
// "A JoLT for the KV cache" (arXiv 2607.12550v4 summary), §3 Method: the
// residual is stored after a feature-axis random orthogonal rotation that is
// seeded, shared by all cells and regenerated at decode.  The library
// regenerates it here, at cache load, from the descriptor's seed:
//   1. SplitMix64 (Steele, Lea and Flood 2014) from `seed`; each 64-bit output
//      x gives the uniform u = ((x >> 11) + 0.5) * 2^-53 in (0, 1);
//   2. Box-Muller on consecutive uniforms (u1, u2): sqrt(-2 ln u1) times
//      (cos 2 pi u2, sin 2 pi u2), filling a d x d matrix Z row by row;
//   3. Householder QR of Z; Pi = Q diag(sign(R_kk)) -- the unique QR factor
//      with a positive-diagonal R, i.e. a Haar-random orthogonal matrix
//      (Mezzadri 2007).
#include <cmath>
#include <cstdint>
#include <vector>

namespace jolt {

// The first n normals of the stream seeded with `seed`: SplitMix64 outputs
// -> uniforms ((x >> 11) + 0.5) 2^-53 -> Box-Muller on consecutive pairs
// (u1, u2): sqrt(-2 ln u1) cos(2 pi u2), then sin(2 pi u2).
void gaussian_fill(uint64_t seed, size_t n, double *out) {
  uint64_t state = seed;
  auto next = [&state]() {
    state += 0x9E3779B97F4A7C15ULL;
    uint64_t z = state;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
  };
  const double two_pi = 2.0 * M_PI;
  for (size_t k = 0; k < n; k += 2) {
    double u1 = ((double)(next() >> 11) + 0.5) * 0x1p-53;
    double u2 = ((double)(next() >> 11) + 0.5) * 0x1p-53;
    double rad = std::sqrt(-2.0 * std::log(u1));
    out[k] = rad * std::cos(two_pi * u2);
    if (k + 1 < n) out[k + 1] = rad * std::sin(two_pi * u2);
  }
}

void make_rotation(uint64_t seed, int d, double *out) {
  const int n = d * d;
  // the Gaussian matrix row by row, then a column-major working copy R[c * d + r]
  std::vector<double> Z(n), R(n);
  gaussian_fill(seed, (size_t)n, Z.data());
  for (int r = 0; r < d; ++r)
    for (int c = 0; c < d; ++c) R[(size_t)c * d + r] = Z[(size_t)r * d + c];
  // Householder: for column k, v = x - alpha e_k with alpha = -sign(x_k)|x|.
  std::vector<double> V((size_t)d * d, 0.0), vn2(d, 0.0), diag(d, 0.0);
  for (int k = 0; k < d; ++k) {
    double *x = &R[(size_t)k * d];
    double nrm2 = 0.0;
    for (int r = k; r < d; ++r) nrm2 += x[r] * x[r];
    double nrm = std::sqrt(nrm2);
    double alpha = x[k] > 0.0 ? -nrm : nrm;
    double *v = &V[(size_t)k * d];
    for (int r = k; r < d; ++r) v[r] = x[r];
    v[k] -= alpha;
    double vv = 0.0;
    for (int r = k; r < d; ++r) vv += v[r] * v[r];
    vn2[k] = vv;
    diag[k] = alpha;
    if (vv == 0.0) continue;
    for (int c = k; c < d; ++c) {
      double *col = &R[(size_t)c * d];
      double dot = 0.0;
      for (int r = k; r < d; ++r) dot += v[r] * col[r];
      double f = 2.0 * dot / vv;
      for (int r = k; r < d; ++r) col[r] -= f * v[r];
    }
  }
  // Q = H_0 H_1 ... H_{d-1} applied to the identity (column-major Q).
  std::vector<double> Q((size_t)d * d, 0.0);
  for (int i = 0; i < d; ++i) Q[(size_t)i * d + i] = 1.0;
  for (int k = d - 1; k >= 0; --k) {
    if (vn2[k] == 0.0) continue;
    const double *v = &V[(size_t)k * d];
    for (int c = 0; c < d; ++c) {
      double *col = &Q[(size_t)c * d];
      double dot = 0.0;
      for (int r = k; r < d; ++r) dot += v[r] * col[r];
      double f = 2.0 * dot / vn2[k];
      for (int r = k; r < d; ++r) col[r] -= f * v[r];
    }
  }
  for (int r = 0; r < d; ++r)
    for (int c = 0; c < d; ++c)
      out[(size_t)r * d + c] = Q[(size_t)c * d + r] * (diag[c] >= 0.0 ? 1.0 : -1.0);
}

}  // namespace jolt
