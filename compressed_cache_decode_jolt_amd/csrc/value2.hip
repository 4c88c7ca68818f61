// Value factors of one query per KV head in a second pass over all heads.
//
// The token factor A_V is shared by every head of a layer ("A JoLT for the
// KV cache" §3: A and B per layer group, G per layer and head), and the value
// side is linear (summary §4.5: dense V is never needed), so with the
// logits of every head at hand the factor-space value sum of all heads is
// one product P A_V -- P [H x T] the softmax weights, A_V [T x r_T] -- which
// reads A_V once per layer instead of once per head and runs on the matrix
// cores.  The split kernel (its logits-out variant) writes the logits and the
// residual part of the output; the merge gives every head's final max m* and
// weight sum L*; then
//   value_gemm:   a[split][h] = sum over the split's tokens of exp(s - m*) A_V[t]
//   value_finish: out[h] += W2_V[h] (sum over splits of a[split][h]) / L*[h]
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "jolt_internal.h"

namespace {

typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 8;  // value_gemm: waves per workgroup, rank blocks dealt round-robin
constexpr int kRB = 4;     // rank blocks of 16 per wave (32 blocks = value ranks up to 512)
constexpr int kUB = 4;     // token blocks whose operands are loaded ahead together

// grid (n2split, nseq): one workgroup per (sequence, token split).  Lane (lr,
// lg) of a wave holds, per 16-token block, the weights of head 16 g + lr for
// tokens 4 lg .. 4 lg + 3 (the B operand of a 16x16x16 product whose K
// dimension is tokens) and the A_V fragment of rank 16 k + lr for the same
// tokens (the A operand, as the value layout stores it); the product
// accumulates a[rank][head] for 16 ranks x 16 heads.  Tokens go in batches of
// kUB blocks.  The weights of a batch are evaluated once per workgroup --
// thread (u, g, lane) turns the four logits of its operand slot into fp16
// exp(s - m*) in an LDS tile -- and every wave reads its B operands there;
// the tile and the waves' A_V fragments are double-buffered, so the next
// batch's logits and fragments are in flight while the current one is
// multiplied, with one barrier per batch.  Logits are stored per 16-token
// block (all heads' 16 logits in turn), so the batch's logits are 8 KiB in
// one piece.
__global__ __launch_bounds__(64 * kWaves) void value_gemm(jolt::V2Args a) {
  static_assert(kUB * 2 * 64 == 64 * kWaves, "one logit operand slot per thread and batch");
  const int split = blockIdx.x, si = blockIdx.y;
  const jolt::SeqV2 &sq = a.seq[si];
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  const int H = a.H, nMV = sq.rT_pad >> 4;  // (> 0: the host sends no rank-0 value factor)
  const int T16 = (sq.T + 15) & ~15;  // the split kernel wrote logits (masked) up to here
  const int t0 = split * a.split2, t1 = min(T16, t0 + a.split2);
  const int ng = H > 16 ? 2 : 1;
  const int nb = t1 > t0 ? (t1 - t0) >> 4 : 0;
  // this thread's operand slot of every batch: block su, head group sg, lane
  // lane (head 16 sg + lr, tokens 4 lg .. 4 lg + 3)
  const int su = tid >> 7, sg = (tid >> 6) & 1, shead = 16 * sg + lr;
  const bool slive = sg < ng && shead < H;
  const float smax = slive ? a.stats[((size_t)sq.slot * H + shead) * 2] : 0.0f;
  const float *sc = a.scores + (size_t)sq.slot * H * a.sc_stride;
  const uint32_t vlane = (uint32_t)lr * 4 + lg;
  __shared__ f16x4 Pt[2][kUB][2][64];  // the weights of a batch, by (block, head group, lane)
  f32x4 acc[kRB][2];
#pragma unroll
  for (int j = 0; j < kRB; ++j)
#pragma unroll
    for (int g = 0; g < 2; ++g) acc[j][g] = f32x4{0, 0, 0, 0};
  f32x4 s4;                // this thread's logits of the next batch
  u32x2 fr[2][kUB][kRB];   // the wave's A_V fragments, per buffer
  // loads of batch b0 (blocks b0 .. b0 + kUB - 1; blocks past the split's
  // end re-read its last block and are not used)
  auto load = [&](int q, int b0) {
    {
      const int tb = t0 + 16 * min(b0 + su, nb - 1);
      s4 = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
      if (slive) s4 = *(const f32x4 *)(sc + ((size_t)(tb >> 4) * H + shead) * 16 + 4 * lg);
    }
#pragma unroll
    for (int u = 0; u < kUB; ++u) {
      const int tb = t0 + 16 * min(b0 + u, nb - 1);
      const uint32_t avb = 2u * ((uint32_t)(tb >> 4) * nMV * 64 + vlane) * 4;
#pragma unroll
      for (int j = 0; j < kRB; ++j) {
        const int k = wave + kWaves * j;
        fr[q][u][j] = ldg<u32x2>(sq.A, avb + 512u * (uint32_t)min(k, nMV - 1));
      }
    }
  };
  auto weights = [&](int q) {
    f16x4 p;
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = (_Float16)__expf(s4[i] - smax);
    Pt[q][su][sg][lane] = p;
  };
  auto compute = [&](int q, int b0) {
#pragma unroll
    for (int u = 0; u < kUB; ++u) {
      if (b0 + u >= nb) break;
      const f16x4 bP0 = Pt[q][u][0][lane];
      const f16x4 bP1 = Pt[q][u][1][lane];
#pragma unroll
      for (int j = 0; j < kRB; ++j) {
        const f16x4 af = __builtin_bit_cast(f16x4, fr[q][u][j]);
        acc[j][0] = __builtin_amdgcn_mfma_f32_16x16x16f16(af, bP0, acc[j][0], 0, 0, 0);
        if (ng > 1) acc[j][1] = __builtin_amdgcn_mfma_f32_16x16x16f16(af, bP1, acc[j][1], 0, 0, 0);
      }
    }
  };
  if (nb > 0) {  // (uniform over the workgroup)
    load(0, 0);
    weights(0);
    __syncthreads();
    for (int b0 = 0; b0 < nb; b0 += 2 * kUB) {
      load(1, b0 + kUB);
      compute(0, b0);
      weights(1);
      __syncthreads();  // tile 1 written; every wave is done with tile 0
      load(0, b0 + 2 * kUB);
      compute(1, b0 + kUB);
      weights(0);
      __syncthreads();
    }
  }
  // lane (lr, lg) holds a[head 16 g + lr][ranks 16 k + 4 lg .. + 3]
  float *pb = a.part + ((size_t)sq.slot * a.n2split + split) * H * a.rV_max;
#pragma unroll
  for (int j = 0; j < kRB; ++j) {
    const int k = wave + kWaves * j;
    if (k >= nMV) continue;
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const int head = 16 * g + lr;
      if (g < ng && head < H) *(f32x4 *)(pb + (size_t)head * a.rV_max + 16 * k + 4 * lg) = acc[j][g];
    }
  }
}

__device__ inline float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

// grid (H, nseq), 512 threads: every output feature f as a wave-wide dot
// product of W2_V row f (lane: 8 ranks) with the splits' summed partial a of
// one (sequence, head), scaled by 1 / L* and added to out.  Thread r first
// loads rank r's partials of the first 16 splits, then wave w issues its 16
// rows 4 w + 32 i + u (i, u < 4) of W2_V, so that the rows are in flight
// while the partials (loaded first, so waited for first) are summed in LDS.
constexpr int kFinWaves = 8;
constexpr int kFinSplits = 16;  // splits whose partials are loaded ahead of W2_V
__global__ __launch_bounds__(64 * kFinWaves) void value_finish(jolt::V2Args a) {
  const int h = blockIdx.x, si = blockIdx.y;
  const jolt::SeqV2 &sq = a.seq[si];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int rV = sq.rT_pad, H = a.H, d = a.d;  // rV <= 512 = the threads, a multiple of 32
  const float *pp = a.part + ((size_t)sq.slot * a.n2split * H + h) * a.rV_max + tid;
  const size_t sstride = (size_t)H * a.rV_max;
  const bool mine = tid < rV;  // this thread sums rank tid
  float pv[kFinSplits];
#pragma unroll
  for (int k = 0; k < kFinSplits; ++k) pv[k] = mine && k < a.n2split ? pp[k * sstride] : 0.0f;
  const _Float16 *W = sq.W2 + (size_t)h * d * rV;
  const int r0 = 8 * lane;  // the lane's ranks r0 .. r0 + 7
  const bool has = r0 < rV;
  f16x8 w[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int f = min(4 * wave + 32 * i + u, d - 1);
      w[i][u] = has ? *(const f16x8 *)(W + (size_t)f * rV + r0) : f16x8{};
    }
  __shared__ float av[512];
  if (mine) {
    float x = 0.0f;
#pragma unroll
    for (int k = 0; k < kFinSplits; ++k) x += pv[k];
    for (int sp = kFinSplits; sp < a.n2split; ++sp) x += pp[sp * sstride];
    av[tid] = x;
  }
  __syncthreads();
  const float inv = 1.0f / a.stats[((size_t)sq.slot * H + h) * 2 + 1];
  float y[8];
  if (has) {
    const f32x4 a0 = *(const f32x4 *)(av + r0), a1 = *(const f32x4 *)(av + r0 + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      y[e] = a0[e];
      y[4 + e] = a1[e];
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      float x = 0.0f;
      if (has)
#pragma unroll
        for (int e = 0; e < 8; ++e) x += (float)w[i][u][e] * y[e];
      x = wave_sum(x);
      const int f = 4 * wave + 32 * i + u;
      if (lane == 0 && f < d) a.out[((size_t)sq.slot * H + h) * d + f] += x * inv;
    }
}

}  // namespace

hipError_t jolt_launch_value2(const jolt::V2Args &a, hipStream_t s, hipEvent_t end) {
  if (a.nseq <= 0) {
    // (a chunk whose second-pass classes had no value factors: the end event
    // still marks the end of the call's work)
    return end ? hipEventRecord(end, s) : hipSuccess;
  }
  hipLaunchKernelGGL(value_gemm, dim3(a.n2split, a.nseq), dim3(64 * kWaves), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (end)
    hipExtLaunchKernelGGL(value_finish, dim3(a.H, a.nseq), dim3(64 * kFinWaves), 0, s, nullptr, end,
                          0u, a);
  else
    hipLaunchKernelGGL(value_finish, dim3(a.H, a.nseq), dim3(64 * kFinWaves), 0, s, a);
  return hipGetLastError();
}
