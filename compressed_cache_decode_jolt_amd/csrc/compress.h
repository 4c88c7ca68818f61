// GPU compressor: kernel launchers shared by compress.hip and compress_host.cpp.
#pragma once
#include <stdint.h>

#include <hip/hip_runtime.h>

namespace jolt {

// One (batched) product C[b] = alpha * sum_k A[b](i, k) B[b](k, j) + beta * D[b](i, j)
// with every operand addressed by element strides:
//   A[b](i, k) = A[b * a_b + i * a_i + k * a_k]   (likewise B, C, D);
// sum_batch = 1 sums the products of all batches into one C (and D) instead.
// Accumulation in float64; C is float64.
struct GemmOp {
  const void *A = nullptr;
  int64_t a_i = 0, a_k = 0, a_b = 0;
  const void *B = nullptr;
  int64_t b_k = 0, b_j = 0, b_b = 0;
  const void *D = nullptr;
  int64_t d_i = 0, d_j = 0, d_b = 0;
  double *C = nullptr;
  int64_t c_i = 0, c_j = 0, c_b = 0;
  int M = 0, N = 0, K = 0, batch = 1, sum_batch = 0;
  double alpha = 1.0, beta = 0.0;
};

// element types of A / B / D: 0 = float64, 1 = float32, 2 = bf16
hipError_t gemm_launch(const GemmOp &g, int ta, int tb, int td, hipStream_t s);
hipError_t quantize_rows_launch(const double *rows, int64_t n, int d, int bits, uint8_t *codes,
                                float *scales, hipStream_t s);
hipError_t round_store_launch(double *x, int64_t n, int bf16, void *out, hipStream_t s);

}  // namespace jolt
