// Internal types shared by the host code and the HIP kernels of libjolt.
//
// Device layout of a loaded cache (private; chosen for gfx950 MFMA operand
// fragments, see the comments on each field).  Notation: H KV heads, d head
// dim, T tokens, T_pad = T rounded up to 128, ranks padded to multiples of 32
// with zeros (a zero rank column contributes nothing to any product).
#pragma once
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "jolt.h"

namespace jolt {

constexpr int kTokPad = 128;    // T padding: one MFMA workgroup tile
constexpr int kRankPad = 32;    // rank padding: one 16x16x32 MFMA K-step
// fp16 elements appended to each row of the key-tile matrices (W2_K, Pi),
// which are copied to LDS as they are.  With rows of 64 k + 32 bytes the
// MFMA operand reads (lane (r, g): row r, 16-byte chunk g) reach the full
// LDS rate on gfx950; strides of 64 k + 16 or 64 k + 48 bytes run at ~57 %
// of it, multiples of 64 far lower (measured with ds_read_b128).
constexpr int kRowPad = 16;
constexpr int kMaxHg = 16;      // query heads per KV head
constexpr int kMaxBatchPerLaunch = 32;
constexpr int kMaxD = 128;
constexpr int kMaxSplits = 2048;
constexpr double kRopeSmall = 128.0;  // radians; see MfmaArgs::rope_small

// Slot order of a 32-deep MFMA K step built from two 16x16 result tiles:
// slot q = 8g + j (g = 16-lane group, j = element of the 8-wide operand)
// holds row perm32(q) of the pair of tiles (lane group g holds rows
// 4g..4g+3 of each).  The key path feeds its rebuilt feature rows to the
// score product in this order, and the queries are laid out to match.
__host__ __device__ inline int perm32(int q) {
  int g = q >> 3, j = q & 7;
  return j < 4 ? 4 * g + j : 16 + 4 * g + (j - 4);
}
__host__ __device__ inline int perm32_inv(int t) {
  if (t < 16) return 8 * (t >> 2) + (t & 3);
  t -= 16;
  return 8 * (t >> 2) + 4 + (t & 3);
}

// Packed-code position of slot q (0..31 within one 32-slot group) for b bits:
// dword q/2/(16/b), bit offset b*((q/2)%(16/b) + (q&1)*(16/b)).  With this
// order one shift and one mask by (2^b-1)|(2^b-1)<<16 place two consecutive
// slots in the two halves of a 32-bit word (two fp16 lanes).
__host__ __device__ inline void code_pos(int q, int bits, int *dword, int *shift) {
  int npair = 16 / bits;
  int P = q >> 1;
  *dword = P / npair;
  *shift = bits * ((P % npair) + (q & 1) * npair);
}

// Value-side layouts follow the operands of a 16x16x16 MFMA whose K
// dimension is 16 tokens: lane (row & 15) * 4 + (t & 15) / 4 holds the four
// consecutive tokens t & ~3 .. (t & ~3) + 3 of one row (a value rank or a
// rotated feature), so a score tile (lane group g holds tokens 4g..4g+3 of
// one query) is the other operand as it stands.
//
// A_V element (t, r): 16 x 16 tiles per (16-token block, 16-rank block).
__host__ __device__ inline size_t av_index(int t, int r, int rT_pad) {
  return (((size_t)(t >> 4) * (rT_pad >> 4) + (r >> 4)) * 64 + (r & 15) * 4 + ((t & 15) >> 2)) * 4 +
         (t & 3);
}
// Value code of (head h, token t, rotated feature f) for b bits and head
// dim d: per (head, 16-token block) 64 lane records of d*b/32 bytes; the
// record of lane (f & 15) * 4 + (t & 15) / 4 holds the d/4 slots
// q = 4 (f / 16) + (t & 3) in code_pos order.  Returns the byte offset of the
// slot's 32-bit word and the bit offset inside it.
__host__ __device__ inline void vcode_pos(int h, int t, int f, int bits, int T_pad, int d,
                                          size_t *byte, int *shift) {
  int dw, sh;
  code_pos(4 * (f >> 4) + (t & 3), bits, &dw, &sh);
  const size_t lane = (size_t)(f & 15) * 4 + ((t & 15) >> 2);
  *byte = (((size_t)h * (T_pad >> 4) + (t >> 4)) * 64 + lane) * (size_t)(d * bits / 32) + 4 * dw;
  *shift = sh;
}

struct CellDev {
  // K: A [T_pad][rT_pad] row-major (fp16, scaled, for bf16 caches).
  // V: A in the av_index layout (factor dtype).
  const void *A;
  // K: G^T of this layer, [H][rF_pad][rT_pad].  V: G of this layer,
  // [H][rT_pad][rF_pad].
  const void *G;
  const void *B;          // [d][rF_pad], factor dtype
  const float *Bt;        // V: B^T as float32, [rF_pad][d] (finalize reads)
  // bf16 caches: W2 = B G[h]^T of this layer, fp16 -- the key tile is
  // rebuilt as W2_K A_K^T in one MFMA chain (keys: [H][d][rT_pad + kRowPad],
  // divided by the A_K scale); for values ([H][d][rT_pad]) it finalizes the
  // split partials.
  const void *W2;
  // Residual codes of this layer.
  // K: [H][T_pad][d*b/8]; a row is 4 chunks (one per 16-lane group g) of
  //    d*b/32 bytes; chunk g holds rotated features i = 32s + 8g + j as slot
  //    q = 8s + j in code_pos order.
  // V: the vcode_pos layout.
  const uint8_t *codes;
  const float *scales;    // this layer: [H][T_pad]
  int32_t rT, rF, bits, rT_pad, rF_pad;
  // Keys of bf16 caches store A as fp16(A * s) with s a power of two (so
  // the MFMA key tile reads A_K rows as they are; W2_K holds B G^T / s);
  // a_inv = 1 / s (1 elsewhere).
  float a_inv;
};

struct LayerDev {
  CellDev c[2];           // [0] = K, [1] = V
  const float *Pi;        // [d][d] float32, row-major
  const float *PiT;       // Pi^T, [d][d] float32 (finalize reads)
  const _Float16 *PiK;    // Pi in fp16, [d][d + kRowPad] (padded rows)
  int32_t T, T_pad, f32;  // f32: factors stored as float32 (else bf16)
};

struct SeqArg {
  const LayerDev *layer;  // device pointer to this sequence's layer descriptor
  int32_t q_pos;
  int32_t T;
  int32_t slot;           // row of this sequence in the launch's q, out and workspace
};

// Kernel arguments of one split-T launch (passed by value, < 4 KiB).
struct DecodeArgs {
  const void *q;          // [batch][H_q][d]
  float *out;             // [batch][H_q][d]
  float *ws;              // partials [batch][H_q][n_split][stride]
  float inv_freq[kMaxD / 2];
  float scale;
  int32_t q_f32, f32;     // f32: the caches store float32 factors
  int32_t H, H_q, Hg, d;
  int32_t n_split, split_tokens, stride, rV_max;
  int32_t nseq;
  SeqArg seq[kMaxBatchPerLaunch];
};

// What the MFMA kernel reads of one sequence's layer: the fields of its
// descriptor copied into the kernel arguments, so that a workgroup's first
// data loads do not wait on a descriptor load.
struct SeqMfma {
  const void *kA, *kcodes, *kW2;
  const float *kscales;
  const void *vA, *vcodes, *vW2;
  const float *vscales;
  const _Float16 *PiK;
  int32_t T, T_pad, q_pos, slot, vrT_pad, pad_;
};

// Kernel arguments of one MFMA split-T launch (passed by value).
struct MfmaArgs {
  const void *q;          // [batch][H_q][d]
  float *ws;              // partials [batch][H_q][n_split][stride]
  float inv_freq[kMaxD / 2];
  float scale;
  int32_t q_f32, H, H_q, Hg;
  int32_t n_split, split_tokens, stride, rV_max, nseq;
  int32_t grid8;          // grid (8 H, n_split / 8, nseq) (n_split % 8 == 0), else (H, n_split, nseq)
  // bit m: every angle t * inv_freq[f] of the launch with 16 m <= f < 16 m + 16
  // is at most kRopeSmall radians (such blocks skip the 2 pi reduction)
  int32_t rope_small;
  SeqMfma seq[kMaxBatchPerLaunch];
};
static_assert(sizeof(MfmaArgs) <= 4096, "MFMA kernel arguments exceed 4 KiB");

// A generic-kernel partial is [m, l, 0, 0, a[rV_max], c[d]] (floats); an
// MFMA-kernel or dense partial is [m, l, 0, 0, o[d]] with o already
// projected to output space and divided by l; m = -inf, l = 0 for an empty
// split.
__host__ __device__ inline int partial_stride(int rV_max, int d) {
  int s = 4 + rV_max + d;
  return (s + 3) & ~3;
}

struct DenseArgs {
  const void *k;          // [batch][H][T][d]
  const void *v;
  const void *q;
  float *out;
  float *ws;              // [batch][H_q][n_split][4 + d]
  float inv_freq[kMaxD / 2];
  float scale;
  int32_t kv_f32, q_f32;
  int32_t batch, H, H_q, Hg, d, T;
  int32_t n_split, split_tokens;
  int32_t q_pos[kMaxBatchPerLaunch];
  int32_t seq0;           // first sequence of this launch
};

}  // namespace jolt

// Global-memory views.  Pointers read from descriptors in memory are
// generic, so without an explicit address space every access would compile
// to a flat load (slower, and it couples the memory and LDS wait counters).
// Native vector types keep small load buffers in registers.
typedef uint32_t gu32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t gu32x2 __attribute__((ext_vector_type(2)));
typedef float gf32x4 __attribute__((ext_vector_type(4)));
template <typename T>
using gptr = const __attribute__((address_space(1))) T *;
template <typename T>
__device__ inline gptr<T> gp(const void *p) {
  return (gptr<T>)p;
}
// Load at a 32-bit byte offset from a uniform base pointer: compiles to a
// global load with the base in scalar registers and one 32-bit offset
// register, with no 64-bit address arithmetic per lane.  Every buffer the
// kernels read this way is smaller than 4 GiB.
template <typename T>
__device__ inline T ldg(const void *base, uint32_t byte_off) {
  return *(gptr<T>)((const __attribute__((address_space(1))) char *)base + byte_off);
}

// Copy rows of 16-byte chunks from global memory to LDS with every thread
// keeping 8 loads in flight (indices are clamped rather than branched on, so
// the loads issue back to back).  src rows are src_cpr chunks long and
// contiguous; dst rows start every dst_stride bytes.
__device__ inline void stage_rows(uint8_t *dst, int dst_stride, const void *src, int rows,
                                  int src_cpr, int tid, int nthreads) {
  const int n = rows * src_cpr;
  if (n <= 0) return;
  gptr<gu32x4> g = gp<gu32x4>(src);
  for (int x0 = 0; x0 < n; x0 += 8 * nthreads) {
    gu32x4 v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int x = x0 + k * nthreads + tid;
      v[k] = g[x < n ? x : n - 1];
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int x = x0 + k * nthreads + tid;
      if (x < n) {
        const int r = x / src_cpr, c = x - r * src_cpr;
        *(gu32x4 *)(dst + (size_t)r * dst_stride + 16 * c) = v[k];
      }
    }
  }
}

namespace jolt {
// Optional timing events of a split-kernel launch: a non-null event is set to
// the launched kernel's own start (begin) or end (end) timestamp.
struct KernelEvents {
  hipEvent_t begin = nullptr, end = nullptr;
};
}  // namespace jolt

// Kernel launchers (kernels_*.hip).  Each returns the hipError_t of its launch.
hipError_t jolt_launch_generic(const jolt::DecodeArgs &a, int nseq, hipStream_t s,
                               jolt::KernelEvents ev);
hipError_t jolt_launch_mfma(const jolt::MfmaArgs &a, int nseq, int bK, int bV, int nkt,
                            int lds_bytes, hipStream_t s, jolt::KernelEvents ev);
hipError_t jolt_launch_merge(const jolt::DecodeArgs &a, int nseq, hipStream_t s);
hipError_t jolt_launch_merge_outputs(const jolt::DecodeArgs &a, int nseq, hipStream_t s);
hipError_t jolt_launch_dense(const jolt::DenseArgs &a, int nseq, hipStream_t s);
hipError_t jolt_launch_dense_merge(const jolt::DenseArgs &a, int nseq, hipStream_t s);
hipError_t jolt_launch_unpack(const jolt::LayerDev *layer, int tau, int H, int T, int d,
                              uint8_t *out, hipStream_t s);
hipError_t jolt_launch_sincos(const float *x, int n, float *sn, float *cs, int variant,
                              hipStream_t s);
int jolt_mfma_max_lds();
