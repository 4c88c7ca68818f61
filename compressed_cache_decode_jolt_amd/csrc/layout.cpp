// Host-side staging of a cache's device image (see layout.h).  Plain C++:
// no HIP runtime, so it also builds for the CPU-only sanitizer check.
#include "layout.h"

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstring>
#include <exception>
#include <mutex>
#include <thread>

namespace jolt {

static inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t Staged::take(size_t bytes) {
  size_t off = buf.size();
  buf.resize(off + align256(bytes), 0);
  return off;
}

static inline float bf16_to_f32(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}
static float load_factor(const void *p, size_t i, bool f32) {
  return f32 ? ((const float *)p)[i] : bf16_to_f32(((const uint16_t *)p)[i]);
}
static void store_factor(uint8_t *dst, size_t i, const void *src, size_t j, bool f32) {
  if (f32)
    ((float *)dst)[i] = ((const float *)src)[j];
  else
    ((uint16_t *)dst)[i] = ((const uint16_t *)src)[j];
}
static inline int canon_code(const uint8_t *row, int i, int bits) {
  int per = 8 / bits;
  return (row[i / per] >> ((i % per) * bits)) & ((1 << bits) - 1);
}

// Runs f(0 .. n-1) on up to `threads` host threads (work items are claimed
// from a shared counter; each item writes a disjoint part of the buffer).
template <class F>
static void parallel_for(int n, int threads, F f) {
  int nt = threads > 0 ? threads : (int)std::max(1u, std::thread::hardware_concurrency());
  nt = std::min(nt, n);
  std::atomic<int> next{0};
  std::exception_ptr err;
  std::mutex mu;
  // an exception in a work item stops the others and is rethrown below, on
  // the calling thread
  auto work = [&] {
    try {
      for (int i; (i = next.fetch_add(1)) < n;) f(i);
    } catch (...) {
      std::lock_guard<std::mutex> g(mu);
      if (!err) err = std::current_exception();
      next.store(n);
    }
  };
  std::vector<std::thread> pool;
  for (int t = 1; t < nt; ++t) {
    try {
      pool.emplace_back(work);
    } catch (...) {
      break;  // fewer threads; the calling thread works too
    }
  }
  work();
  for (auto &th : pool) th.join();
  if (err) std::rethrow_exception(err);
}

void stage_cache(const jolt_cache_desc *desc, Staged *S, int threads) {
  const int H = desc->n_kv_heads, d = desc->head_dim, T = desc->T;
  const bool f32 = desc->factor_dtype == JOLT_F32;
  const int fb = f32 ? 4 : 2;
  const int T_pad = (T + kTokPad - 1) / kTokPad * kTokPad;
  const int n_groups = desc->n_groups;
  S->T_pad = T_pad;

  std::vector<double> Pi64((size_t)d * d);
  make_rotation(desc->rotation_seed, d, Pi64.data());
  S->off_pi = S->take(sizeof(float) * d * d);
  for (int i = 0; i < d * d; ++i) ((float *)(S->buf.data() + S->off_pi))[i] = (float)Pi64[i];
  S->off_pit = S->take(sizeof(float) * d * d);
  for (int r = 0; r < d; ++r)
    for (int c = 0; c < d; ++c)
      ((float *)(S->buf.data() + S->off_pit))[(size_t)c * d + r] = (float)Pi64[(size_t)r * d + c];
  // Pi in fp16 with padded rows: the MFMA kernel copies it to LDS as it is
  const int pik_row = d + kRowPad;
  S->off_pik = S->take(sizeof(_Float16) * d * pik_row);
  for (int r = 0; r < d; ++r)
    for (int c = 0; c < d; ++c)
      ((_Float16 *)(S->buf.data() + S->off_pik))[(size_t)r * pik_row + c] = (_Float16)Pi64[(size_t)r * d + c];

  S->cells.assign(2 * n_groups, CellMeta{});
  S->offs.assign(2 * n_groups, CellOffsets{});
  for (int g = 0; g < n_groups; ++g) {
    const int gs = desc->group_start[g + 1] - desc->group_start[g];
    for (int tau = 0; tau < 2; ++tau) {
      const jolt_cell &in = desc->cells[2 * g + tau];
      CellMeta m;
      m.rT = in.r_T;
      m.rF = in.r_F;
      m.bits = in.bits;
      m.rT_pad = pad_rank(in.r_T);
      m.rF_pad = (in.r_F + kRankPad - 1) / kRankPad * kRankPad;
      CellOffsets &o = S->offs[2 * g + tau];
      // A (keys in the ak_index layout, values in av_index).  bf16 caches:
      // fp16 scaled by a power of two a_s (exact for every
      // bf16 value in fp16's normal range) so that the MFMA products take A
      // as it is -- A_K fragments in the key tile, A_V against fp16 softmax
      // weights (11-bit, where bf16 weights would carry 8); W2 carries the
      // 1 / a_s.
      o.A = S->take((size_t)fb * T_pad * std::max(m.rT_pad, 1));
      m.a_s = 1.0;
      if (!f32) {
        float amax = 0.0f;
        for (size_t i = 0; i < (size_t)T * m.rT; ++i)
          amax = std::max(amax, std::fabs(load_factor(in.A, i, false)));
        if (amax > 0.0f) {
          int E;
          std::frexp(amax, &E);  // amax in [2^(E-1), 2^E)
          m.a_s = std::ldexp(1.0, 8 - E);
        }
      }
      for (int t = 0; t < T; ++t)
        for (int r = 0; r < m.rT; ++r) {
          const size_t dst = tau == 0 ? ak_index(t, r, m.rT_pad) : av_index(t, r, m.rT_pad);
          if (!f32)
            ((_Float16 *)(S->buf.data() + o.A))[dst] =
                (_Float16)(load_factor(in.A, (size_t)t * m.rT + r, false) * (float)m.a_s);
          else
            store_factor(S->buf.data() + o.A, dst, in.A, (size_t)t * m.rT + r, true);
        }
      // B, and B^T in float32 for the value finalize of the float32 kernel
      o.B = S->take((size_t)fb * d * std::max(m.rF_pad, 1));
      for (int f = 0; f < d; ++f)
        for (int j = 0; j < m.rF; ++j)
          store_factor(S->buf.data() + o.B, (size_t)f * m.rF_pad + j, in.B, (size_t)f * m.rF + j, f32);
      o.Bt = S->take(sizeof(float) * std::max(m.rF_pad, 1) * d);
      for (int f = 0; f < d; ++f)
        for (int j = 0; j < m.rF; ++j)
          ((float *)(S->buf.data() + o.Bt))[(size_t)j * d + f] = load_factor(in.B, (size_t)f * m.rF + j, f32);
      // per layer of the group: reserve G, W2, codes and scales first (the
      // buffer must not move while threads fill it)
      const bool w2 = !f32 && m.rT > 0;
      const int w2_row = m.rT_pad + (tau == 0 ? kRowPad : 0);  // key rows padded like their LDS image
      const int rowb = m.bits ? d * m.bits / 8 : 0;
      for (int lp = 0; lp < gs; ++lp) {
        o.G.push_back(S->take((size_t)fb * H * std::max(m.rT_pad, 1) * std::max(m.rF_pad, 1)));
        o.W2.push_back(w2 ? S->take(sizeof(uint16_t) * H * d * w2_row) : 0);
        o.codes.push_back(m.bits ? S->take((size_t)H * T_pad * rowb) : 0);
        o.scales.push_back(m.bits ? S->take(sizeof(float) * H * T_pad) : 0);
      }
      S->cells[2 * g + tau] = m;
      std::vector<double> Bf;
      if (w2) {
        Bf.resize((size_t)d * m.rF);
        for (size_t i = 0; i < Bf.size(); ++i) Bf[i] = load_factor(in.B, i, false);
      }
      uint8_t *base = S->buf.data();
      // one work item per (layer of the group, head)
      parallel_for(gs * H, threads, [&](int item) {
        const int lp = item / H, h = item % H;
        uint8_t *Gd = base + o.G[lp];
        for (int r = 0; r < m.rT; ++r)
          for (int j = 0; j < m.rF; ++j) {
            const size_t src = (((size_t)lp * H + h) * m.rT + r) * m.rF + j;
            const size_t dst = tau == 0 ? ((size_t)h * m.rF_pad + j) * m.rT_pad + r
                                        : ((size_t)h * m.rT_pad + r) * m.rF_pad + j;
            store_factor(Gd, dst, in.G, src, f32);
          }
        // W2[h] = B G[lp, h]^T / a_s (bf16 caches): key-tile matrix and
        // value-finalize matrix, fp16, formed in float64 and rounded once
        if (w2) {
          _Float16 *W2 = (_Float16 *)(base + o.W2[lp]);
          std::vector<double> Gf((size_t)m.rT * m.rF);
          for (size_t i = 0; i < Gf.size(); ++i)
            Gf[i] = load_factor(in.G, ((size_t)lp * H + h) * m.rT * m.rF + i, false);
          for (int f = 0; f < d; ++f)
            for (int r = 0; r < m.rT; ++r) {
              double acc = 0.0;
              for (int j = 0; j < m.rF; ++j) acc += Bf[(size_t)f * m.rF + j] * Gf[(size_t)r * m.rF + j];
              W2[((size_t)h * d + f) * w2_row + r] = (_Float16)(acc / m.a_s);
            }
        }
        if (m.bits == 0) return;
        const int b = m.bits;
        uint8_t *C = base + o.codes[lp];
        float *Sc = (float *)(base + o.scales[lp]);
        for (int t = 0; t < T; ++t) {
          const uint8_t *row = in.codes + (((size_t)lp * H + h) * T + t) * rowb;
          Sc[(size_t)h * T_pad + t] = in.scales[((size_t)lp * H + h) * T + t];
          for (int i = 0; i < d; ++i) {
            const uint32_t code = (uint32_t)canon_code(row, i, b);
            size_t at;
            int sh;
            if (tau == 0)
              kcode_pos(h, t, i, b, T_pad, d, &at, &sh);
            else
              vcode_pos(h, t, i, b, T_pad, d, &at, &sh);
            uint32_t w;
            std::memcpy(&w, C + at, 4);
            w |= code << sh;
            std::memcpy(C + at, &w, 4);
          }
        }
      });
    }
  }
}

}  // namespace jolt
