// Device layout of a loaded cache: index maps and the host-side staging of
// one cache's device image.  Plain C++ (no HIP runtime), so the re-layout can
// be built and checked on a CPU alone, under the address and undefined-
// behaviour sanitizers; the kernels include the same index maps through
// jolt_internal.h.
//
// Notation: H KV heads, d head dim, T tokens, T_pad = T rounded up to 128,
// ranks padded to multiples of 32 with zeros (a zero rank column contributes
// nothing to any product).
#pragma once
#include <stddef.h>
#include <stdint.h>

#include <vector>

#include "jolt.h"

#if defined(__HIPCC__)
#define JOLT_HD __host__ __device__
#else
#define JOLT_HD
#endif

namespace jolt {

constexpr int kTokPad = 128;    // T padding: one MFMA workgroup tile
constexpr int kRankPad = 32;    // rank padding: one 16x16x32 MFMA K-step
// fp16 elements appended to each row of the key-tile matrices (W2_K, Pi),
// which are copied to LDS as they are.  With rows of 64 k + 32 bytes the
// MFMA operand reads (lane (r, g): row r, 16-byte chunk g) reach the full
// LDS rate on gfx950; strides of 64 k + 16 or 64 k + 48 bytes run at ~57 %
// of it, multiples of 64 far lower (measured with ds_read_b128).
constexpr int kRowPad = 16;

// Slot order of a 32-deep MFMA K step built from two 16x16 result tiles:
// slot q = 8g + j (g = 16-lane group, j = element of the 8-wide operand)
// holds row perm32(q) of the pair of tiles (lane group g holds rows
// 4g..4g+3 of each).  The key path feeds its rebuilt feature rows to the
// score product in this order, and the queries are laid out to match.
JOLT_HD inline int perm32(int q) {
  int g = q >> 3, j = q & 7;
  return j < 4 ? 4 * g + j : 16 + 4 * g + (j - 4);
}
JOLT_HD inline int perm32_inv(int t) {
  if (t < 16) return 8 * (t >> 2) + (t & 3);
  t -= 16;
  return 8 * (t >> 2) + 4 + (t & 3);
}

// Packed-code position of slot q (0..31 within one 32-slot group) for b bits:
// dword q/2/(16/b), bit offset b*((q/2)%(16/b) + (q&1)*(16/b)).  With this
// order one shift and one mask by (2^b-1)|(2^b-1)<<16 place two consecutive
// slots in the two halves of a 32-bit word (two fp16 lanes).
JOLT_HD inline void code_pos(int q, int bits, int *dword, int *shift) {
  int npair = 16 / bits;
  int P = q >> 1;
  *dword = P / npair;
  *shift = bits * ((P % npair) + (q & 1) * npair);
}

// Key residual codes: a (head, token) row has d*b/8 bytes in 4 chunks of
// d*b/32 bytes, one per 16-lane group g of the MFMA operand; chunk g holds
// rotated feature i = 32 s + 8 g + j as slot q = 8 s + j in code_pos order.
// Per 16-token block of a head, the lanes (t & 15, g) read their chunks as
// pieces of at most 16 bytes; piece x of every lane sits in one contiguous
// run of 64 pieces (lane (t & 15) * 4 + g at 16 bytes each), so a wave load
// of a piece reads contiguous bytes.  Chunks of 16 bytes or less are one
// piece, and the block is then simply its 16 rows in order.
JOLT_HD inline void kcode_pos(int h, int t, int i, int bits, int T_pad, int d, size_t *byte,
                              int *shift) {
  int dw, sh;
  code_pos(8 * (i >> 5) + (i & 7), bits, &dw, &sh);
  const int cb = d * bits / 32, pc = cb < 16 ? cb : 16;  // chunk, piece bytes
  const int x = 4 * dw / pc, in = 4 * dw - x * pc;       // piece, byte in it
  *byte = ((size_t)h * T_pad + (t & ~15)) * (size_t)(d * bits / 8) + (size_t)x * 64 * pc +
          (size_t)((t & 15) * 4 + ((i >> 3) & 3)) * pc + in;
  *shift = sh;
}

// A_K element (t, r): one B operand of the key tile's 16x16x32 MFMA -- 16
// tokens x 32 ranks, 1 KiB in fp16 -- per (16-token block, 32-rank step),
// blocks outermost; lane (t & 15) * 4 + ((r >> 3) & 3) of the operand holds
// ranks 8 ((r >> 3) & 3) .. + 7 of token t, so one wave load of a step reads
// one contiguous KiB (8 whole cache lines, where token rows would touch 16
// half lines).  rT_pad is a multiple of 32.
JOLT_HD inline size_t ak_index(int t, int r, int rT_pad) {
  return (((size_t)(t >> 4) * (rT_pad >> 5) + (r >> 5)) * 64 + (t & 15) * 4 + ((r >> 3) & 3)) * 8 +
         (r & 7);
}

// Value-side layouts follow the operands of a 16x16x16 MFMA whose K
// dimension is 16 tokens: lane (row & 15) * 4 + (t & 15) / 4 holds the four
// consecutive tokens t & ~3 .. (t & ~3) + 3 of one row (a value rank or a
// rotated feature), so a score tile (lane group g holds tokens 4g..4g+3 of
// one query) is the other operand as it stands.
//
// A_V element (t, r): 16 x 16 tiles per (16-token block, 16-rank block).
JOLT_HD inline size_t av_index(int t, int r, int rT_pad) {
  return (((size_t)(t >> 4) * (rT_pad >> 4) + (r >> 4)) * 64 + (r & 15) * 4 + ((t & 15) >> 2)) * 4 +
         (t & 3);
}
// Value code of (head h, token t, rotated feature f) for b bits and head
// dim d: per (head, 16-token block) 64 lane records of d*b/32 bytes; the
// record of lane (f & 15) * 4 + (t & 15) / 4 holds the d/4 slots
// q = 4 (f / 16) + (t & 3) in code_pos order.  Returns the byte offset of the
// slot's 32-bit word and the bit offset inside it.
JOLT_HD inline void vcode_pos(int h, int t, int f, int bits, int T_pad, int d, size_t *byte,
                              int *shift) {
  int dw, sh;
  code_pos(4 * (f >> 4) + (t & 3), bits, &dw, &sh);
  const size_t lane = (size_t)(f & 15) * 4 + ((t & 15) >> 2);
  *byte = (((size_t)h * (T_pad >> 4) + (t >> 4)) * 64 + lane) * (size_t)(d * bits / 32) + 4 * dw;
  *shift = sh;
}

// Padded rank of a cell: multiples of 32; ranks above 256 pad to 64, so wide
// key tiles take an even number of 32-rank MFMA steps.
// LDS of one MFMA decode workgroup, byte offsets into its dynamic LDS.  The
// host sizes the launch with .total and the kernel places its arrays at these
// offsets, so the two cannot disagree.
//   kt: key-rank blocks of 32; nmv: value-rank blocks of 16; pi_lds: Pi's
//   fp16 image sits in LDS next to W2_K; hg1v: the one-query-per-KV-head
//   kernel variant (parks 4 lanes' f16x4 per value block instead of 64).
// During the token-block loop: W2_K (+ Pi) at [0, kpath), the softmax (m, l)
// exchange, the frequencies, the query operands (and their low halves with
// more than 8 queries per KV head) and the block counter.  After it the
// parked value partials take [0, park) and the combined value tiles Xa / Xc
// go behind them when they fit below kpath (one-query variant only), else
// behind the query operands.
struct MfmaLds {
  uint32_t kpath, park, red, ifr, qf, ql, xa, xa_bytes, ctr, total;
  bool xa_r0;
};
JOLT_HD constexpr MfmaLds mfma_lds_layout(int d, int kt, bool pi_lds, int nmv, int waves,
                                          bool hg1v) {
  MfmaLds l{};
  l.kpath = 2u * d * (32 * kt + kRowPad) + (pi_lds ? 2u * d * (d + kRowPad) : 0u);
  l.park = (uint32_t)waves * (nmv + 8) * (hg1v ? 4 : 64) * 8;
  l.xa_bytes = (uint32_t)(nmv + 8) * 64 * 16;
  l.xa_r0 = hg1v && l.park + l.xa_bytes <= l.kpath;
  l.red = l.xa_r0 || l.kpath > l.park ? l.kpath : l.park;
  l.ifr = l.red + 2u * 16 * waves * 4;   // [2][waves][16] floats
  l.qf = l.ifr + 2u * 64 * 4;            // [2][64] floats
  l.ql = l.qf + 4u * 96 * 16;            // [4 K-steps][16][6] f16x8
  l.xa = l.xa_r0 ? l.park : l.ql;        // low halves alias Xa: Xa is written after the loop
  // the counter is live during the loop: never inside [0, kpath) or Ql
  l.ctr = l.xa_r0 ? l.ql : l.xa + l.xa_bytes;
  l.total = l.ctr + 16;
  return l;
}

inline int pad_rank(int r) {
  const int m = r > 8 * kRankPad ? 2 * kRankPad : kRankPad;
  return (r + m - 1) / m * m;
}

struct CellMeta {
  int rT, rF, bits, rT_pad, rF_pad;
  double a_s;  // bf16 caches: A stored as fp16(A * a_s), a_s a power of two
};

// Byte offsets, inside one staging buffer, of a cell's sections (per layer
// of its group where the section is per layer; 0 = absent).
struct CellOffsets {
  size_t A = 0, B = 0, Bt = 0;
  std::vector<size_t> G, W2, codes, scales;
};

// The device image of one cache, built in host memory: one buffer that is
// copied to a single device allocation as it is.  Sections start at
// 256-byte boundaries.
//   Pi fp32 [d][d], Pi^T fp32 [d][d], PiK fp16 [d][d + kRowPad];
//   per cell: A -- keys [T_pad][rT_pad] (fp16 A*a_s for bf16 caches, fp32
//   otherwise), values in the av_index layout; B [d][rF_pad] (factor dtype);
//   B^T fp32 [rF_pad][d]; per layer: G (K: [H][rF_pad][rT_pad], V:
//   [H][rT_pad][rF_pad]), W2 = B G[h]^T / a_s fp16 for bf16 caches (keys
//   [H][d][rT_pad + kRowPad], values [H][d][rT_pad]), codes (K: kcode_pos,
//   V: vcode_pos layout) and scales fp32 [H][T_pad].
struct Staged {
  std::vector<uint8_t> buf;
  int T_pad = 0;
  size_t off_pi = 0, off_pit = 0, off_pik = 0;
  std::vector<CellMeta> cells;      // [n_groups * 2]
  std::vector<CellOffsets> offs;    // [n_groups * 2]
  size_t take(size_t bytes);        // append a zeroed, 256-aligned section
};

// Fill *out from a descriptor that has passed validation.  Regenerates Pi
// from the seed, re-lays out A, B, G, W2, codes and scales.  Throws
// std::bad_alloc when host memory runs out.  Uses up to `threads` host
// threads (0 = all hardware threads).
void stage_cache(const jolt_cache_desc *desc, Staged *out, int threads = 0);

void make_rotation(uint64_t seed, int d, double *out);
void gaussian_fill(uint64_t seed, size_t n, double *out);

}  // namespace jolt
