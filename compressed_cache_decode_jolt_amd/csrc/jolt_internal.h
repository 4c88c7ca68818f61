// Internal types shared by the host code and the HIP kernels of libjolt.
//
// Device layout of a loaded cache (private; chosen for gfx950 MFMA operand
// fragments, see the comments on each field and layout.h for the index
// maps).  Notation: H KV heads, d head dim, T tokens, T_pad = T rounded up to
// 128, ranks padded to multiples of 32 with zeros.
#pragma once
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "jolt.h"
#include "layout.h"  // constants and index maps of the device layout

namespace jolt {

constexpr int kMaxHg = 16;      // query heads per KV head
constexpr int kMaxBatchPerLaunch = 32;
constexpr int kMaxD = 128;
constexpr int kMaxSplits = 2048;
constexpr int kMaxTailSplits = 256;  // splits of an uncompressed tail
constexpr double kRopeSmall = 128.0;  // radians; see MfmaArgs::rope_small

// Whether a launch with one query per KV head runs the one-query (HG1)
// variant of its class -- key bits, value bits, key-rank steps of 32 and
// value-rank blocks of 16 (after padding): the wide-key classes (4 waves)
// and the value-rank-above-128 classes (8 waves), except 8-bit keys and
// values with 8 key-rank steps, whose 8-wave variant does not fit its
// registers and which runs the grouped-query 4-wave class instead.  The
// launcher and the host's LDS sizing both follow this.
__host__ __device__ constexpr bool hg1_variant(int bK, int bV, int kt, int nmv) {
  return kt > 8 || (nmv > 8 && !(bK == 8 && bV == 8 && kt == 8));
}

// One query per KV head with key ranks above 256 (kt > 8) and value ranks
// above 128: the logits-out variant (the value factors in a second pass over
// all heads) runs 8 waves with Pi in LDS where W2_K and Pi fit there -- d =
// 128; with a key residual that is key ranks up to 448.
__host__ __device__ constexpr bool wide_sco(int bK, int kt) {
  return kt > 8 && mfma_lds_layout(128, kt, bK > 0, 0, 8, true).total <= 160u * 1024u;
}

struct CellDev {
  // K: A [T_pad][rT_pad] in MFMA operand fragments (ak_index layout; fp16,
  // scaled, for bf16 caches).
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
  // the MFMA key tile reads A_K fragments as they are; W2_K holds B G^T / s);
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
  // uncompressed-tail partials of the float32 path, [batch][H_q][n_tsplit][4 + d]
  // (dense layout; n_tsplit = 0: no tail)
  const float *tail_ws;
  int32_t n_tsplit;
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
  float *ws;              // partials [batch][H_q][ws_splits][stride] (this launch: the first n_split)
  float inv_freq[kMaxD / 2];
  float scale;
  int32_t q_f32, H, H_q, Hg;
  int32_t n_split, split_tokens, stride, rV_max, nseq;
  int32_t ws_splits;      // splits per (sequence, query head) row of ws (>= n_split)
  int32_t grid8;          // 1: grid (8 H, n_split / 8, nseq) (n_split % 8 == 0); 2: (8 H, nseq
                          // n_split / 8, 1) (nseq n_split % 8 == 0); 0: (H, n_split, nseq)
  // bit m: every angle t * inv_freq[f] of the launch with 16 m <= f < 16 m + 16
  // is at most kRopeSmall radians (such blocks skip the 2 pi reduction)
  int32_t rope_small;
  // 1: fixed token-block schedule (wave w takes blocks w, w + waves, ...),
  // bitwise reproducible; 0: blocks claimed on demand
  int32_t fixed_blocks;
  // one query per KV head, value factors in a second pass (the split kernel
  // variant with SCO): every token's logit goes to scores, laid out
  // [slot][sc_stride / 16][H][16] (per 16-token block, the 16 logits of every
  // head in turn), and the split partials carry the residual part only
  float *scores;
  int32_t sc_stride;
  // one split per (sequence, KV head) and no tail (nothing to merge): when
  // out is set, the kernel writes each query head's output o / l to
  // out[(slot H_q + query head) d + f] instead of a partial, and, when stats
  // is set, its (max, weight sum) to stats[(slot H_q + query head) 2 + 0/1]
  float *out;
  float *stats;
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
  float *ws;              // [batch][H_q][ws_splits][4 + d]; this launch's splits start at split0
  float inv_freq[kMaxD / 2];
  float scale;
  int32_t kv_f32, q_f32;
  int32_t batch, H, H_q, Hg, d, T;  // T: rows per (sequence, head) in k and v
  int32_t n_split, split_tokens;
  int32_t ws_splits, split0;
  int32_t q_pos[kMaxBatchPerLaunch];
  int32_t T_seq[kMaxBatchPerLaunch];  // tokens of each sequence (<= T) that are attended to
  int32_t seq0;           // first sequence of this launch
};

// Second pass of the value factors for one query per KV head (value_gemm /
// value_finish): a[h] = sum_t exp(s[h, t] - m*[h]) A_V[t] over all heads at
// once, then out[h] += W2_V[h] a[h] / L*[h].
struct SeqV2 {
  const void *A;         // A_V, fp16 (A_V s), 16 x 16 tiles (av_index layout)
  const _Float16 *W2;    // W2_V [H][d][rT_pad] fp16
  int32_t T, rT_pad, slot, pad_;
};
struct V2Args {
  const float *scores;   // logits [slot][sc_stride / 16][H][16]
  const float *stats;    // (m*, L*) [slot][H][2] from the merge
  float *part;           // [slot][n2split][H][rV_max] partial a
  float *out;            // [slot][H][d], the merge's output, a-part added
  int32_t H, d, sc_stride, n2split, split2, rV_max, nseq;
  SeqV2 seq[kMaxBatchPerLaunch];
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
// stats (may be NULL): (max, sum of weights) per (sequence, query head)
hipError_t jolt_launch_merge_outputs(const jolt::DecodeArgs &a, int nseq, int ns, hipStream_t s,
                                     float *stats = nullptr);
// end (may be NULL): set to the end time of the pass's last kernel
hipError_t jolt_launch_value2(const jolt::V2Args &a, hipStream_t s, hipEvent_t end);
hipError_t jolt_launch_dense(const jolt::DenseArgs &a, int nseq, hipStream_t s);
hipError_t jolt_launch_dense_merge(const jolt::DenseArgs &a, int nseq, hipStream_t s);
hipError_t jolt_launch_unpack(const jolt::LayerDev *layer, int tau, int H, int T, int d,
                              uint8_t *out, hipStream_t s);
hipError_t jolt_launch_sincos(const float *x, int n, float *sn, float *cs, int variant,
                              hipStream_t s);
int jolt_mfma_max_lds();
