// GPU compressor (FlashJoLT) -- host orchestration of compress.hip.
//
// "A JoLT for the KV cache" (arXiv 2607.12550v4 summary), §3 Method and §3.1
// "Fast variant: FlashJoLT": partial Tucker decomposition of a grouped cache
// by ST-HOSVD whose token-mode SVD is a randomized low-rank SVD of the
// leading q_cap directions (randomized subspace iteration, Halko, Martinsson
// and Tropp 2011, Algorithms 4.4 and 5.1), the exact feature-mode SVD, the
// residual against the stored factors, rotated by the seeded Pi, quantised
// to b bits and packed; for the allocator, the q_cap token-mode energies plus
// one synthetic tail entry (the norm's remainder), the feature-mode energies
// and the squared norm.
//
// Every product runs in the GEMM kernel of compress.hip (float64
// accumulation); the k x k and d x d factorisations (Cholesky, triangular
// inverse, symmetric eigendecomposition; k = q_cap + oversample, a few
// hundred at most) use rocSOLVER on the same stream.  orth() is CholeskyQR2
// -- Q of the QR factorisation with a positive diagonal in R -- with a shifted
// first pass when the Gram matrix is numerically singular.
#include <hip/hip_runtime.h>
#include <rocblas/rocblas.h>
#include <rocsolver/rocsolver.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <string>
#include <vector>

#include "compress.h"
#include "errors.h"
#include "jolt.h"
#include "layout.h"

using namespace jolt;

namespace {

struct DevMem {
  void *p = nullptr;
  ~DevMem() {
    if (p) (void)hipFree(p);
  }
  template <typename T>
  T *get() const {
    return (T *)p;
  }
};

struct Ctx {
  hipStream_t s = nullptr;
  rocblas_handle h = nullptr;
  std::string err;
  ~Ctx() {
    if (h) rocblas_destroy_handle(h);
  }
};

#define CK(expr)                                                          \
  do {                                                                    \
    hipError_t e_ = (expr);                                               \
    if (e_ != hipSuccess) {                                               \
      cx.err = std::string(#expr) + ": " + hipGetErrorString(e_);         \
      return false;                                                       \
    }                                                                     \
  } while (0)
#define CKR(expr)                                                         \
  do {                                                                    \
    rocblas_status r_ = (expr);                                           \
    if (r_ != rocblas_status_success) {                                   \
      cx.err = std::string(#expr) + ": " + rocblas_status_to_string(r_);  \
      return false;                                                       \
    }                                                                     \
  } while (0)

bool dalloc(Ctx &cx, DevMem &m, size_t bytes) {
  CK(hipMalloc(&m.p, std::max<size_t>(bytes, 256)));
  return true;
}

bool gemm(Ctx &cx, const GemmOp &g, int ta = 0, int tb = 0, int td = 0) {
  CK(gemm_launch(g, ta, tb, td, cx.s));
  return true;
}

// C (n x n) = Y^T Y for Y (m x n) row-major
bool gram(Ctx &cx, const double *Y, int64_t m, int n, double *C) {
  GemmOp g;
  g.A = Y, g.a_i = 1, g.a_k = n;
  g.B = Y, g.b_k = n, g.b_j = 1;
  g.C = C, g.c_i = n, g.c_j = 1;
  g.M = n, g.N = n, g.K = (int)m;
  return gemm(cx, g);
}

bool read_info(Ctx &cx, const int *d_info, int *h_info) {
  CK(hipMemcpyAsync(h_info, d_info, sizeof(int), hipMemcpyDeviceToHost, cx.s));
  CK(hipStreamSynchronize(cx.s));
  return true;
}

// Y (m x n, row-major, device) <- Q of Y = Q R with diag(R) > 0, by
// CholeskyQR2 (a shifted first pass if Y^T Y is numerically singular).
// tmp: m x n scratch; C: n x n scratch; info: device int.
bool orth(Ctx &cx, double *&Y, double *&tmp, int64_t m, int n, double *C, int *info) {
  int passes = 2;
  for (int p = 0; p < passes; ++p) {
    if (!gram(cx, Y, m, n, C)) return false;
    // rocSOLVER works column-major; the Gram matrix is symmetric, so its
    // upper triangle is the same either way
    CKR(rocsolver_dpotrf(cx.h, rocblas_fill_upper, n, C, n, info));
    int hinfo = 0;
    if (!read_info(cx, info, &hinfo)) return false;
    if (hinfo != 0) {
      if (p > 0) {
        cx.err = "CholeskyQR: Gram matrix not positive definite after a shifted pass";
        return false;
      }
      // shifted pass (Fukaya et al. 2020): C + s I with s ~ 11 (m n + n (n + 1)) u ||Y||^2
      if (!gram(cx, Y, m, n, C)) return false;
      std::vector<double> hc((size_t)n * n);
      CK(hipMemcpyAsync(hc.data(), C, sizeof(double) * n * n, hipMemcpyDeviceToHost, cx.s));
      CK(hipStreamSynchronize(cx.s));
      double tr = 0.0;
      for (int i = 0; i < n; ++i) tr += hc[(size_t)i * n + i];
      const double shift = 11.0 * ((double)m * n + (double)n * (n + 1)) * 1.1102230246251565e-16 * tr;
      for (int i = 0; i < n; ++i) hc[(size_t)i * n + i] += shift;
      CK(hipMemcpyAsync(C, hc.data(), sizeof(double) * n * n, hipMemcpyHostToDevice, cx.s));
      CKR(rocsolver_dpotrf(cx.h, rocblas_fill_upper, n, C, n, info));
      if (!read_info(cx, info, &hinfo)) return false;
      if (hinfo != 0) {
        cx.err = "CholeskyQR: shifted Gram matrix not positive definite";
        return false;
      }
      passes = 3;
    }
    CKR(rocsolver_dtrtri(cx.h, rocblas_fill_upper, rocblas_diagonal_non_unit, n, C, n, info));
    // Y R^{-1}: R^{-1} upper triangular, column-major (element (r, c) at r + c n),
    // entries below the diagonal are left from the Gram matrix and skipped
    // by zeroing them first
    {
      std::vector<double> hc((size_t)n * n);
      CK(hipMemcpyAsync(hc.data(), C, sizeof(double) * n * n, hipMemcpyDeviceToHost, cx.s));
      CK(hipStreamSynchronize(cx.s));
      for (int c = 0; c < n; ++c)
        for (int r = c + 1; r < n; ++r) hc[(size_t)r + (size_t)c * n] = 0.0;
      CK(hipMemcpyAsync(C, hc.data(), sizeof(double) * n * n, hipMemcpyHostToDevice, cx.s));
    }
    GemmOp g;
    g.A = Y, g.a_i = n, g.a_k = 1;
    g.B = C, g.b_k = 1, g.b_j = n;
    g.C = tmp, g.c_i = n, g.c_j = 1;
    g.M = (int)m, g.N = n, g.K = n;
    if (!gemm(cx, g)) return false;
    std::swap(Y, tmp);
  }
  return true;
}

// Symmetric eigendecomposition of the n x n device matrix S (overwritten by
// the eigenvectors, column-major, eigenvalues ascending into host w).
bool eigh(Ctx &cx, double *S, int n, std::vector<double> &w, int *info) {
  DevMem dD, dE;
  if (!dalloc(cx, dD, sizeof(double) * n) || !dalloc(cx, dE, sizeof(double) * n)) return false;
  CKR(rocsolver_dsyevd(cx.h, rocblas_evect_original, rocblas_fill_upper, n, S, n, dD.get<double>(),
                       dE.get<double>(), info));
  int hinfo = 0;
  if (!read_info(cx, info, &hinfo)) return false;
  if (hinfo != 0) {
    cx.err = "symmetric eigensolver did not converge";
    return false;
  }
  w.resize(n);
  CK(hipMemcpyAsync(w.data(), dD.p, sizeof(double) * n, hipMemcpyDeviceToHost, cx.s));
  CK(hipStreamSynchronize(cx.s));
  return true;
}

struct Shape {
  int gs, H, T, d, tx;  // tx: element type of X (1 = float32, 2 = bf16)
  int64_t nb() const { return (int64_t)gs * H; }
  int64_t N() const { return nb() * d; }
};

// Z (N x k) = M^T Q for the token unfolding M of X and Q (T x k).
bool unfold_t_times(Ctx &cx, const Shape &sh, const void *X, const double *Q, int k, double *Z) {
  GemmOp g;
  g.A = X, g.a_i = 1, g.a_k = sh.d, g.a_b = (int64_t)sh.T * sh.d;
  g.B = Q, g.b_k = k, g.b_j = 1, g.b_b = 0;
  g.C = Z, g.c_i = k, g.c_j = 1, g.c_b = (int64_t)sh.d * k;
  g.M = sh.d, g.N = k, g.K = sh.T, g.batch = (int)sh.nb();
  return gemm(cx, g, sh.tx, 0, 0);
}
// Y (T x k) = M W for W (N x k).
bool unfold_times(Ctx &cx, const Shape &sh, const void *X, const double *W, int k, double *Y) {
  GemmOp g;
  g.A = X, g.a_i = sh.d, g.a_k = 1, g.a_b = (int64_t)sh.T * sh.d;
  g.B = W, g.b_k = k, g.b_j = 1, g.b_b = (int64_t)sh.d * k;
  g.C = Y, g.c_i = k, g.c_j = 1;
  g.M = sh.T, g.N = k, g.K = sh.d, g.batch = (int)sh.nb(), g.sum_batch = 1;
  return gemm(cx, g, sh.tx, 0, 0);
}

// Randomized token basis: U (T x q, device, row-major) and the q leading
// singular values (host, descending).
bool token_basis(Ctx &cx, const Shape &sh, const void *X, const jolt_flash_params &fp, DevMem &U,
                 int *q_out, std::vector<double> &sig) {
  const int64_t T = sh.T, N = sh.N();
  const int k = (int)std::min<int64_t>({(int64_t)fp.q_cap + fp.oversample, T, N});
  const int q = std::min(fp.q_cap, k);
  DevMem dOm, dY, dT1, dZ, dZt, dC, dInfo;
  if (!dalloc(cx, dOm, sizeof(double) * N * k) || !dalloc(cx, dY, sizeof(double) * T * k) ||
      !dalloc(cx, dT1, sizeof(double) * T * k) || !dalloc(cx, dZ, sizeof(double) * N * k) ||
      !dalloc(cx, dZt, sizeof(double) * N * k) || !dalloc(cx, dC, sizeof(double) * k * k) ||
      !dalloc(cx, dInfo, sizeof(int)))
    return false;
  {
    std::vector<double> om((size_t)N * k);
    gaussian_fill(fp.sketch_seed, om.size(), om.data());
    CK(hipMemcpyAsync(dOm.p, om.data(), sizeof(double) * om.size(), hipMemcpyHostToDevice, cx.s));
    CK(hipStreamSynchronize(cx.s));
  }
  double *Y = dY.get<double>(), *T1 = dT1.get<double>(), *Z = dZ.get<double>(), *Zt = dZt.get<double>();
  int *info = dInfo.get<int>();
  if (!unfold_times(cx, sh, X, dOm.get<double>(), k, Y)) return false;
  if (!orth(cx, Y, T1, T, k, dC.get<double>(), info)) return false;
  for (int it = 0; it < fp.power_iters; ++it) {
    if (!unfold_t_times(cx, sh, X, Y, k, Z)) return false;
    if (!orth(cx, Z, Zt, N, k, dC.get<double>(), info)) return false;
    if (!unfold_times(cx, sh, X, Z, k, Y)) return false;
    if (!orth(cx, Y, T1, T, k, dC.get<double>(), info)) return false;
  }
  // Q^T M = Z^T with Z = M^T Q; its left singular vectors are the
  // eigenvectors of Z^T Z
  if (!unfold_t_times(cx, sh, X, Y, k, Z)) return false;
  if (!gram(cx, Z, N, k, dC.get<double>())) return false;
  std::vector<double> w;
  if (!eigh(cx, dC.get<double>(), k, w, info)) return false;
  // U = Q V[:, top q] (eigenvector columns taken in descending order)
  if (!dalloc(cx, U, sizeof(double) * T * q)) return false;
  GemmOp g;
  g.A = Y, g.a_i = k, g.a_k = 1;
  g.B = dC.get<double>() + (size_t)(k - 1) * k, g.b_k = 1, g.b_j = -(int64_t)k;
  g.C = U.get<double>(), g.c_i = q, g.c_j = 1;
  g.M = (int)T, g.N = q, g.K = k;
  if (!gemm(cx, g)) return false;
  sig.resize(q);
  for (int c = 0; c < q; ++c) sig[c] = std::sqrt(std::max(w[k - 1 - c], 0.0));
  *q_out = q;
  return true;
}

// d x d Gram matrix of the feature unfolding of X (sum over layers, heads and
// tokens) and its eigenvalues, descending; ||X||^2 is its trace.
bool feature_gram(Ctx &cx, const Shape &sh, const void *X, std::vector<double> &ev, double *norm2) {
  const int d = sh.d;
  DevMem dF, dInfo;
  if (!dalloc(cx, dF, sizeof(double) * d * d) || !dalloc(cx, dInfo, sizeof(int))) return false;
  GemmOp g;
  g.A = X, g.a_i = 1, g.a_k = d, g.a_b = (int64_t)sh.T * d;
  g.B = X, g.b_k = d, g.b_j = 1, g.b_b = (int64_t)sh.T * d;
  g.C = dF.get<double>(), g.c_i = d, g.c_j = 1;
  g.M = d, g.N = d, g.K = sh.T, g.batch = (int)sh.nb(), g.sum_batch = 1;
  if (!gemm(cx, g, sh.tx, sh.tx, 0)) return false;
  std::vector<double> F((size_t)d * d);
  CK(hipMemcpyAsync(F.data(), dF.p, sizeof(double) * d * d, hipMemcpyDeviceToHost, cx.s));
  CK(hipStreamSynchronize(cx.s));
  double tr = 0.0;
  for (int i = 0; i < d; ++i) tr += F[(size_t)i * d + i];
  *norm2 = tr;
  std::vector<double> w;
  if (!eigh(cx, dF.get<double>(), d, w, dInfo.get<int>())) return false;
  ev.resize(d);
  for (int i = 0; i < d; ++i) ev[i] = std::max(w[d - 1 - i], 0.0);
  return true;
}

bool check_shape(const void *X, jolt_dtype xt, int gs, int H, int T, int d,
                 const jolt_flash_params *p, std::string *why) {
  if (!X || !p) return *why = "NULL X or params", false;
  if (xt != JOLT_F32 && xt != JOLT_BF16) return *why = "X dtype", false;
  if (gs < 1 || H < 1 || T < 1 || d < 2 || d > 128) return *why = "shape", false;
  if (p->q_cap < 1 || p->oversample < 0 || p->power_iters < 0 || p->power_iters > 16)
    return *why = "flash params", false;
  if ((int64_t)p->q_cap + p->oversample > 4096) return *why = "q_cap + oversample > 4096", false;
  if ((int64_t)gs * H * T > (int64_t)1 << 26 || T > (1 << 22)) return *why = "cell too large", false;
  return true;
}

}  // namespace

extern "C" jolt_status jolt_flash_spectra(const void *X, jolt_dtype x_dtype, int32_t group_size,
                                          int32_t n_kv_heads, int32_t T, int32_t head_dim,
                                          const jolt_flash_params *p, double *sT2, double *sF2,
                                          double *norm2, jolt_stream stream) {
  return jolt::guarded("jolt_flash_spectra", [&]() -> jolt_status {
    std::string why;
    if (!check_shape(X, x_dtype, group_size, n_kv_heads, T, head_dim, p, &why))
      return set_error(JOLT_E_INVALID, "jolt_flash_spectra: %s", why.c_str());
    if (!sT2 || !sF2 || !norm2) return set_error(JOLT_E_INVALID, "NULL output");
    Ctx cx;
    cx.s = (hipStream_t)stream;
    if (rocblas_create_handle(&cx.h) != rocblas_status_success)
      return set_error(JOLT_E_HIP, "rocblas_create_handle failed");
    rocblas_set_stream(cx.h, cx.s);
    const Shape sh{group_size, n_kv_heads, T, head_dim, x_dtype == JOLT_F32 ? 1 : 2};
    DevMem U;
    int q = 0;
    std::vector<double> sig, ev;
    double n2 = 0.0;
    if (!token_basis(cx, sh, X, *p, U, &q, sig) || !feature_gram(cx, sh, X, ev, &n2))
      return set_error(JOLT_E_HIP, "jolt_flash_spectra: %s", cx.err.c_str());
    double acc = 0.0;
    for (int i = 0; i < p->q_cap; ++i) {
      const double v = i < q ? sig[i] * sig[i] : 0.0;
      sT2[i] = v;
      acc += v;
    }
    sT2[p->q_cap] = std::max(n2 - acc, 0.0);
    for (int i = 0; i < head_dim; ++i) sF2[i] = ev[i];
    *norm2 = n2;
    return set_error(JOLT_OK, "");
  });
}

extern "C" jolt_status jolt_flash_compress_cell(
    const void *X, jolt_dtype x_dtype, int32_t group_size, int32_t n_kv_heads, int32_t T,
    int32_t head_dim, const jolt_flash_params *p, int32_t r_T, int32_t r_F, int32_t bits,
    uint64_t rotation_seed, jolt_dtype factor_dtype, void *A, void *B, void *G, uint8_t *codes,
    float *scales, jolt_stream stream) {
  return jolt::guarded("jolt_flash_compress_cell", [&]() -> jolt_status {
    std::string why;
    if (!check_shape(X, x_dtype, group_size, n_kv_heads, T, head_dim, p, &why))
      return set_error(JOLT_E_INVALID, "jolt_flash_compress_cell: %s", why.c_str());
    const int d = head_dim;
    if (r_T < 0 || r_F < 0 || r_F > d || (r_T == 0) != (r_F == 0) ||
        r_T > std::min<int64_t>(T, (int64_t)group_size * n_kv_heads * d))
      return set_error(JOLT_E_INVALID, "ranks r_T=%d r_F=%d", r_T, r_F);
    if (r_T > p->q_cap) return set_error(JOLT_E_INVALID, "r_T=%d above q_cap=%d", r_T, p->q_cap);
    if (bits != 0 && bits != 2 && bits != 4 && bits != 8)
      return set_error(JOLT_E_INVALID, "bits=%d", bits);
    if (factor_dtype != JOLT_F32 && factor_dtype != JOLT_BF16)
      return set_error(JOLT_E_INVALID, "factor dtype");
    if (r_T > 0 && (!A || !B || !G)) return set_error(JOLT_E_INVALID, "NULL factor output");
    if (bits > 0 && (!codes || !scales)) return set_error(JOLT_E_INVALID, "NULL code output");
    if (bits > 0 && (d * bits) % 8) return set_error(JOLT_E_INVALID, "d * bits not a byte multiple");

    Ctx cx;
    cx.s = (hipStream_t)stream;
    if (rocblas_create_handle(&cx.h) != rocblas_status_success)
      return set_error(JOLT_E_HIP, "rocblas_create_handle failed");
    rocblas_set_stream(cx.h, cx.s);
    const Shape sh{group_size, n_kv_heads, T, d, x_dtype == JOLT_F32 ? 1 : 2};
    const int64_t nb = sh.nb();
    const int fbytes = factor_dtype == JOLT_BF16 ? 2 : 4;
    const int bf = factor_dtype == JOLT_BF16 ? 1 : 0;
    auto run = [&]() -> bool {
      DevMem dA, dB, dG, dSa, dSb, dSg, dW, dInfo;
      if (!dalloc(cx, dInfo, sizeof(int))) return false;
      if (r_T > 0) {
        DevMem U, dYp, dF;
        int q = 0;
        std::vector<double> sig;
        if (!token_basis(cx, sh, X, *p, U, &q, sig)) return false;
        // A = U[:, :r_T]
        if (!dalloc(cx, dA, sizeof(double) * T * r_T)) return false;
        CK(hipMemcpy2DAsync(dA.p, sizeof(double) * r_T, U.p, sizeof(double) * q, sizeof(double) * r_T,
                            T, hipMemcpyDeviceToDevice, cx.s));
        // Y[l, h] = A^T X[l, h]  (r_T x d)
        if (!dalloc(cx, dYp, sizeof(double) * nb * r_T * d)) return false;
        GemmOp g;
        g.A = dA.p, g.a_i = 1, g.a_k = r_T, g.a_b = 0;
        g.B = X, g.b_k = d, g.b_j = 1, g.b_b = (int64_t)T * d;
        g.C = dYp.get<double>(), g.c_i = d, g.c_j = 1, g.c_b = (int64_t)r_T * d;
        g.M = r_T, g.N = d, g.K = T, g.batch = (int)nb;
        if (!gemm(cx, g, 0, sh.tx, 0)) return false;
        // feature basis: leading r_F eigenvectors of sum_lh Y^T Y
        if (!dalloc(cx, dF, sizeof(double) * d * d)) return false;
        g = GemmOp();
        g.A = dYp.p, g.a_i = 1, g.a_k = d, g.a_b = (int64_t)r_T * d;
        g.B = dYp.p, g.b_k = d, g.b_j = 1, g.b_b = (int64_t)r_T * d;
        g.C = dF.get<double>(), g.c_i = d, g.c_j = 1;
        g.M = d, g.N = d, g.K = r_T, g.batch = (int)nb, g.sum_batch = 1;
        if (!gemm(cx, g)) return false;
        std::vector<double> w;
        if (!eigh(cx, dF.get<double>(), d, w, dInfo.get<int>())) return false;
        std::vector<double> V((size_t)d * d), hB((size_t)d * r_F);
        CK(hipMemcpyAsync(V.data(), dF.p, sizeof(double) * d * d, hipMemcpyDeviceToHost, cx.s));
        CK(hipStreamSynchronize(cx.s));
        for (int f = 0; f < d; ++f)
          for (int c = 0; c < r_F; ++c) hB[(size_t)f * r_F + c] = V[(size_t)f + (size_t)(d - 1 - c) * d];
        if (!dalloc(cx, dB, sizeof(double) * d * r_F)) return false;
        CK(hipMemcpyAsync(dB.p, hB.data(), sizeof(double) * hB.size(), hipMemcpyHostToDevice, cx.s));
        // G[l, h] = Y[l, h] B  (r_T x r_F)
        if (!dalloc(cx, dG, sizeof(double) * nb * r_T * r_F)) return false;
        g = GemmOp();
        g.A = dYp.p, g.a_i = d, g.a_k = 1, g.a_b = (int64_t)r_T * d;
        g.B = dB.p, g.b_k = r_F, g.b_j = 1, g.b_b = 0;
        g.C = dG.get<double>(), g.c_i = r_F, g.c_j = 1, g.c_b = (int64_t)r_T * r_F;
        g.M = r_T, g.N = r_F, g.K = d, g.batch = (int)nb;
        if (!gemm(cx, g)) return false;
        // round to the storage dtype (in place) and keep the stored bits
        const int64_t nA = (int64_t)T * r_T, nB = (int64_t)d * r_F, nG = nb * r_T * r_F;
        if (!dalloc(cx, dSa, fbytes * nA) || !dalloc(cx, dSb, fbytes * nB) || !dalloc(cx, dSg, fbytes * nG))
          return false;
        CK(round_store_launch(dA.get<double>(), nA, bf, dSa.p, cx.s));
        CK(round_store_launch(dB.get<double>(), nB, bf, dSb.p, cx.s));
        CK(round_store_launch(dG.get<double>(), nG, bf, dSg.p, cx.s));
        CK(hipMemcpyAsync(A, dSa.p, fbytes * nA, hipMemcpyDeviceToHost, cx.s));
        CK(hipMemcpyAsync(B, dSb.p, fbytes * nB, hipMemcpyDeviceToHost, cx.s));
        CK(hipMemcpyAsync(G, dSg.p, fbytes * nG, hipMemcpyDeviceToHost, cx.s));
        if (bits > 0) {
          // W[l, h] = G_s[l, h] B_s^T  (r_T x d)
          if (!dalloc(cx, dW, sizeof(double) * nb * r_T * d)) return false;
          g = GemmOp();
          g.A = dG.p, g.a_i = r_F, g.a_k = 1, g.a_b = (int64_t)r_T * r_F;
          g.B = dB.p, g.b_k = 1, g.b_j = r_F, g.b_b = 0;
          g.C = dW.get<double>(), g.c_i = d, g.c_j = 1, g.c_b = (int64_t)r_T * d;
          g.M = r_T, g.N = d, g.K = r_F, g.batch = (int)nb;
          if (!gemm(cx, g)) return false;
        }
      }
      if (bits > 0) {
        // R[l, h] = X[l, h] - A_s W[l, h], then R' = R Pi, then codes
        const int64_t rows = nb * T;
        DevMem dR, dRp, dPi, dCodes, dScales;
        if (!dalloc(cx, dR, sizeof(double) * rows * d) || !dalloc(cx, dRp, sizeof(double) * rows * d) ||
            !dalloc(cx, dPi, sizeof(double) * d * d) || !dalloc(cx, dCodes, rows * d * bits / 8) ||
            !dalloc(cx, dScales, sizeof(float) * rows))
          return false;
        GemmOp g;
        g.A = r_T > 0 ? dA.p : nullptr, g.a_i = r_T, g.a_k = 1, g.a_b = 0;
        g.B = r_T > 0 ? dW.p : nullptr, g.b_k = d, g.b_j = 1, g.b_b = (int64_t)r_T * d;
        g.D = X, g.d_i = d, g.d_j = 1, g.d_b = (int64_t)T * d;
        g.C = dR.get<double>(), g.c_i = d, g.c_j = 1, g.c_b = (int64_t)T * d;
        g.M = T, g.N = d, g.K = r_T, g.batch = (int)nb;
        g.alpha = -1.0, g.beta = 1.0;
        if (!gemm(cx, g, 0, 0, sh.tx)) return false;
        std::vector<double> Pi((size_t)d * d);
        make_rotation(rotation_seed, d, Pi.data());
        CK(hipMemcpyAsync(dPi.p, Pi.data(), sizeof(double) * d * d, hipMemcpyHostToDevice, cx.s));
        // R' = R Pi over all rows, in chunks the grid can hold
        const int64_t chunk = (int64_t)60000 * 64;
        for (int64_t r0 = 0; r0 < rows; r0 += chunk) {
          g = GemmOp();
          g.A = dR.get<double>() + r0 * d, g.a_i = d, g.a_k = 1;
          g.B = dPi.p, g.b_k = d, g.b_j = 1;
          g.C = dRp.get<double>() + r0 * d, g.c_i = d, g.c_j = 1;
          g.M = (int)std::min(chunk, rows - r0), g.N = d, g.K = d;
          if (!gemm(cx, g)) return false;
        }
        CK(quantize_rows_launch(dRp.get<double>(), rows, d, bits, dCodes.get<uint8_t>(),
                                dScales.get<float>(), cx.s));
        CK(hipMemcpyAsync(codes, dCodes.p, rows * d * bits / 8, hipMemcpyDeviceToHost, cx.s));
        CK(hipMemcpyAsync(scales, dScales.p, sizeof(float) * rows, hipMemcpyDeviceToHost, cx.s));
        CK(hipStreamSynchronize(cx.s));
      }
      CK(hipStreamSynchronize(cx.s));
      return true;
    };
    if (!run()) return set_error(JOLT_E_HIP, "jolt_flash_compress_cell: %s", cx.err.c_str());
    return set_error(JOLT_OK, "");
  });
}

// Alignment-based layer grouping ("A JoLT for the KV cache" §3): each
// layer's token basis U_l (T x r) from the randomized SVD of its keys and
// values side by side, the alignment ||U_l^T U_{l+1}||_F^2 / r of neighbours,
// and groups = maximal runs of neighbours aligned at least tau (at most
// max_group layers each, 0 = no limit).
extern "C" jolt_status jolt_flash_layer_groups(const void *const *k_layers,
                                               const void *const *v_layers, jolt_dtype x_dtype,
                                               int32_t n_layers, int32_t n_kv_heads, int32_t T,
                                               int32_t head_dim, const jolt_flash_params *p,
                                               double tau, int32_t max_group,
                                               int32_t *group_start, int32_t *n_groups,
                                               double *align, jolt_stream stream) {
  return jolt::guarded("jolt_flash_layer_groups", [&]() -> jolt_status {
    std::string why;
    if (!k_layers || !v_layers || !group_start || !n_groups || n_layers < 1 || max_group < 0 ||
        std::isnan(tau))
      return set_error(JOLT_E_INVALID, "jolt_flash_layer_groups: bad arguments");
    for (int l = 0; l < n_layers; ++l)
      if (!check_shape(k_layers[l], x_dtype, 2, n_kv_heads, T, head_dim, p, &why) || !v_layers[l])
        return set_error(JOLT_E_INVALID, "jolt_flash_layer_groups: layer %d: %s", l,
                         why.empty() ? "NULL values" : why.c_str());
    Ctx cx;
    cx.s = (hipStream_t)stream;
    if (rocblas_create_handle(&cx.h) != rocblas_status_success)
      return set_error(JOLT_E_HIP, "rocblas_create_handle failed");
    rocblas_set_stream(cx.h, cx.s);
    const int eb = x_dtype == JOLT_F32 ? 4 : 2;
    const size_t half = (size_t)n_kv_heads * T * head_dim * eb;
    const Shape sh{2, n_kv_heads, T, head_dim, x_dtype == JOLT_F32 ? 1 : 2};
    std::vector<double> a(n_layers > 1 ? n_layers - 1 : 0);
    auto run = [&]() -> bool {
      DevMem dX, dC, prevU;
      int prev_q = 0;
      if (!dalloc(cx, dX, 2 * half)) return false;
      for (int l = 0; l < n_layers; ++l) {
        // keys then values of the layer, contiguous: [2][H][T][d]
        CK(hipMemcpyAsync(dX.p, k_layers[l], half, hipMemcpyDeviceToDevice, cx.s));
        CK(hipMemcpyAsync((uint8_t *)dX.p + half, v_layers[l], half, hipMemcpyDeviceToDevice, cx.s));
        DevMem U;
        int q = 0;
        std::vector<double> sig;
        if (!token_basis(cx, sh, dX.p, *p, U, &q, sig)) return false;
        if (l > 0) {
          if (!dC.p && !dalloc(cx, dC, sizeof(double) * q * q)) return false;
          GemmOp g;
          g.A = prevU.p, g.a_i = 1, g.a_k = prev_q;
          g.B = U.p, g.b_k = q, g.b_j = 1;
          g.C = dC.get<double>(), g.c_i = q, g.c_j = 1;
          g.M = prev_q, g.N = q, g.K = T;
          if (!gemm(cx, g)) return false;
          std::vector<double> hc((size_t)prev_q * q);
          CK(hipMemcpyAsync(hc.data(), dC.p, sizeof(double) * hc.size(), hipMemcpyDeviceToHost, cx.s));
          CK(hipStreamSynchronize(cx.s));
          double ss = 0.0;
          for (double v : hc) ss += v * v;
          a[l - 1] = ss / prev_q;
        }
        std::swap(prevU.p, U.p);
        prev_q = q;
      }
      return true;
    };
    if (!run()) return set_error(JOLT_E_HIP, "jolt_flash_layer_groups: %s", cx.err.c_str());
    int ng = 0;
    group_start[0] = 0;
    for (int l = 1; l < n_layers; ++l) {
      const int size = l - group_start[ng];
      if (a[l - 1] < tau || (max_group > 0 && size >= max_group)) group_start[++ng] = l;
    }
    group_start[++ng] = n_layers;
    *n_groups = ng;
    if (align)
      for (int l = 0; l + 1 < n_layers; ++l) align[l] = a[l];
    return set_error(JOLT_OK, "");
  });
}

extern "C" jolt_status jolt_quantize_rows(const double *rows, int64_t n_rows, int32_t d, int32_t bits,
                                          uint8_t *codes, float *scales, jolt_stream stream) {
  if (n_rows < 0 || d < 2 || d > 128 || (bits != 2 && bits != 4 && bits != 8) || (d * bits) % 8)
    return set_error(JOLT_E_INVALID, "jolt_quantize_rows: n_rows=%lld d=%d bits=%d",
                     (long long)n_rows, d, bits);
  if (n_rows > 0 && (!rows || !codes || !scales)) return set_error(JOLT_E_INVALID, "NULL pointer");
  hipError_t e = quantize_rows_launch(rows, n_rows, d, bits, codes, scales, (hipStream_t)stream);
  if (e != hipSuccess) return set_error(JOLT_E_HIP, "quantize launch: %s", hipGetErrorString(e));
  return set_error(JOLT_OK, "");
}
