// GPU compressor kernels (FlashJoLT): the products of the randomized
// token-mode SVD and of the ST-HOSVD that follows it, factor rounding to the
// storage dtype, and the rotated residual's quantiser and packer.
//
// "A JoLT for the KV cache" (arXiv 2607.12550v4 summary), §3 (partial Tucker
// by ST-HOSVD, rotated residual quantised to b bits) and §3.1 "Fast variant:
// FlashJoLT" (randomized token-mode SVD).  Every product here accumulates in
// float64: the compressor runs once per prefill, off the decode clock, and
// float64 keeps its factors within rounding of the exact decomposition.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "compress.h"

namespace jolt {
namespace {

template <typename T>
__device__ inline double ld(const void *p, int64_t i);
template <>
__device__ inline double ld<double>(const void *p, int64_t i) {
  return ((const double *)p)[i];
}
template <>
__device__ inline double ld<float>(const void *p, int64_t i) {
  return (double)((const float *)p)[i];
}
template <>
__device__ inline double ld<uint16_t>(const void *p, int64_t i) {  // bf16 bits
  return (double)__uint_as_float((uint32_t)((const uint16_t *)p)[i] << 16);
}

// C = alpha op(A) op(B) + beta D, all addressed by element strides (see
// GemmOp).  64 x 64 output tile per workgroup of 256 threads, 4 x 4 outputs
// per thread, K in chunks of 16 staged in LDS; float64 accumulation.
constexpr int kTile = 64, kChunk = 16;

template <typename TA, typename TB, typename TD>
__global__ __launch_bounds__(256) void gemm64(GemmOp g) {
  __shared__ double As[kChunk][kTile + 1];
  __shared__ double Bs[kChunk][kTile + 1];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int i0 = blockIdx.y * kTile, j0 = blockIdx.x * kTile;
  double acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = 0.0;
  const int b_lo = g.sum_batch ? 0 : blockIdx.z, b_hi = g.sum_batch ? g.batch : blockIdx.z + 1;
  for (int bb = b_lo; bb < b_hi; ++bb) {
    const int64_t abase = (int64_t)bb * g.a_b, bbase = (int64_t)bb * g.b_b;
    for (int k0 = 0; k0 < g.K; k0 += kChunk) {
      // stage A[i0 .. i0+63][k0 .. k0+15] and B[k0 .. k0+15][j0 .. j0+63]
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int e = tid + 256 * r;          // 0 .. 1023
        const int kk = e & 15, ii = e >> 4;   // A: consecutive threads walk k
        const int gi = i0 + ii, gk = k0 + kk;
        As[kk][ii] = (gi < g.M && gk < g.K) ? ld<TA>(g.A, abase + gi * g.a_i + gk * g.a_k) : 0.0;
        const int jj = e & 63, kb = e >> 6;   // B: consecutive threads walk j
        const int gj = j0 + jj, gk2 = k0 + kb;
        Bs[kb][jj] = (gj < g.N && gk2 < g.K) ? ld<TB>(g.B, bbase + gk2 * g.b_k + gj * g.b_j) : 0.0;
      }
      __syncthreads();
#pragma unroll
      for (int kk = 0; kk < kChunk; ++kk) {
        double av[4], bv[4];
#pragma unroll
        for (int a = 0; a < 4; ++a) av[a] = As[kk][ty + 16 * a];
#pragma unroll
        for (int b = 0; b < 4; ++b) bv[b] = Bs[kk][tx + 16 * b];
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
          for (int b = 0; b < 4; ++b) acc[a][b] = fma(av[a], bv[b], acc[a][b]);
      }
      __syncthreads();
    }
  }
  const int cb = g.sum_batch ? 0 : blockIdx.z;
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int i = i0 + ty + 16 * a, j = j0 + tx + 16 * b;
      if (i < g.M && j < g.N) {
        double v = g.alpha * acc[a][b];
        if (g.D) v += g.beta * ld<TD>(g.D, (int64_t)cb * g.d_b + i * g.d_i + j * g.d_j);
        g.C[(int64_t)cb * g.c_b + i * g.c_i + j * g.c_j] = v;
      }
    }
}

// Quantise and pack rotated residual rows (one 64-lane wave per row):
//   delta = fl32(2 max_i |r_i| / L),  c_i = clip(rint(r_i / delta + L/2), 0, L)
// (ties to even), delta = 0 -> c_i = floor(L/2); codes packed least
// significant bits first into d*b/8 bytes.  The decisions are taken in
// float64 from the float64 rows.
__global__ __launch_bounds__(256) void quantize_rows_kernel(const double *rows, int64_t n, int d,
                                                            int bits, uint8_t *codes, float *scales) {
  __shared__ uint8_t cbuf[4][128];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + wave;
  if (row >= n) return;
  const double *r = rows + row * d;
  const int L = (1 << bits) - 1;
  const double x0 = lane < d ? r[lane] : 0.0, x1 = lane + 64 < d ? r[lane + 64] : 0.0;
  double m = fmax(fabs(x0), fabs(x1));
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmax(m, __shfl_xor(m, o));
  const float delta = (float)(2.0 * m / (double)L);
  const double dd = (double)delta;
  auto code = [&](double x) -> int {
    if (dd == 0.0) return L / 2;
    double c = rint(x / dd + (double)L / 2.0);
    c = fmin(fmax(c, 0.0), (double)L);
    return (int)c;
  };
  if (lane < d) cbuf[wave][lane] = (uint8_t)code(x0);
  if (lane + 64 < d) cbuf[wave][lane + 64] = (uint8_t)code(x1);
  if (lane == 0) scales[row] = delta;
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const int nbytes = d * bits / 8, per = 8 / bits;
  for (int bidx = lane; bidx < nbytes; bidx += 64) {
    uint32_t v = 0;
    for (int e = 0; e < per; ++e) v |= (uint32_t)cbuf[wave][bidx * per + e] << (e * bits);
    codes[row * nbytes + bidx] = (uint8_t)v;
  }
}

// Round float64 values to the storage dtype: writes the rounded value back
// as float64 (for the reconstruction the residual is taken against) and the
// stored bits (bf16: float64 -> float32 -> bf16, each round-to-nearest-even).
__global__ void round_store_kernel(double *x, int64_t n, int bf16, void *out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const float f = (float)x[i];
  if (bf16) {
    uint32_t u = __float_as_uint(f);
    u = (u + 0x7FFFu + ((u >> 16) & 1u)) & 0xFFFF0000u;
    ((uint16_t *)out)[i] = (uint16_t)(u >> 16);
    x[i] = (double)__uint_as_float(u);
  } else {
    ((float *)out)[i] = f;
    x[i] = (double)f;
  }
}

}  // namespace

template <typename TA, typename TB, typename TD>
static hipError_t launch(const GemmOp &g, hipStream_t s) {
  dim3 grid((unsigned)((g.N + kTile - 1) / kTile), (unsigned)((g.M + kTile - 1) / kTile),
            (unsigned)(g.sum_batch ? 1 : g.batch));
  hipLaunchKernelGGL((gemm64<TA, TB, TD>), grid, dim3(256), 0, s, g);
  return hipGetLastError();
}

// ta / tb / td: 0 = float64, 1 = float32, 2 = bf16
hipError_t gemm_launch(const GemmOp &g, int ta, int tb, int td, hipStream_t s) {
  if (g.M <= 0 || g.N <= 0 || g.batch <= 0) return hipSuccess;
  if (ta == 0 && tb == 0 && td == 0) return launch<double, double, double>(g, s);
  if (ta == 1 && tb == 0 && td == 0) return launch<float, double, double>(g, s);
  if (ta == 2 && tb == 0 && td == 0) return launch<uint16_t, double, double>(g, s);
  if (ta == 0 && tb == 1 && td == 0) return launch<double, float, double>(g, s);
  if (ta == 0 && tb == 2 && td == 0) return launch<double, uint16_t, double>(g, s);
  if (ta == 1 && tb == 1 && td == 0) return launch<float, float, double>(g, s);
  if (ta == 2 && tb == 2 && td == 0) return launch<uint16_t, uint16_t, double>(g, s);
  if (ta == 0 && tb == 0 && td == 1) return launch<double, double, float>(g, s);
  if (ta == 0 && tb == 0 && td == 2) return launch<double, double, uint16_t>(g, s);
  return hipErrorInvalidValue;
}

hipError_t quantize_rows_launch(const double *rows, int64_t n, int d, int bits, uint8_t *codes,
                                float *scales, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(quantize_rows_kernel, dim3((unsigned)((n + 3) / 4)), dim3(256), 0, s, rows, n,
                     d, bits, codes, scales);
  return hipGetLastError();
}

hipError_t round_store_launch(double *x, int64_t n, int bf16, void *out, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(round_store_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, x, n,
                     bf16, out);
  return hipGetLastError();
}

}  // namespace jolt
