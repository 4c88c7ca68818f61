// Host side of libjolt: argument validation, error reporting, cache upload
// and re-layout, and kernel dispatch.  Every entry point is declared, with
// its contract, in include/jolt.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "jolt.h"
#include "jolt_internal.h"

namespace jolt {
void make_rotation(uint64_t seed, int d, double *out);
}

using namespace jolt;

// RoPE angles t * inv_freq are evaluated by a reduction valid below 2^20 rad
// (trig.h): positions are limited to 2^20 and frequencies to [0, 1].
static constexpr int kMaxPos = 1 << 20;

static jolt_status check_rope(const int32_t *q_pos, int batch, const float *inv_freq, int d) {
  for (int b = 0; b < batch; ++b)
    if (q_pos[b] < 0 || q_pos[b] > kMaxPos)
      return JOLT_E_INVALID;
  for (int i = 0; i < d / 2; ++i)
    if (!(inv_freq[i] >= 0.0f && inv_freq[i] <= 1.0f)) return JOLT_E_INVALID;
  return JOLT_OK;
}

// ---------------------------------------------------------------- errors --
static thread_local std::string g_err;

static jolt_status fail(jolt_status st, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}
static jolt_status ok() {
  g_err.clear();
  return JOLT_OK;
}

#define HIP_TRY(expr)                                                               \
  do {                                                                              \
    hipError_t e_ = (expr);                                                         \
    if (e_ != hipSuccess) return fail(JOLT_E_HIP, "%s: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

extern "C" const char *jolt_last_error(void) { return g_err.c_str(); }

// ------------------------------------------------------------- helpers --
static inline int round_up(int x, int m) { return (x + m - 1) / m * m; }
static inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

static inline float bf16_to_f32(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

// --------------------------------------------------------- cache handle --
struct CellMeta {
  int rT, rF, bits, rT_pad, rF_pad;
  double a_s;  // bf16 caches: A stored as fp16(A * a_s)
};

struct jolt_cache {
  int n_layers = 0, n_groups = 0, H = 0, H_q = 0, d = 0, T = 0, T_pad = 0;
  bool f32 = false;
  int device = 0;
  std::vector<int> group_start;
  std::vector<CellMeta> cells;      // [n_groups * 2]
  std::vector<int> layer_group;     // [n_layers]
  void *dev = nullptr;
  size_t dev_bytes = 0;
  LayerDev *d_layers = nullptr;     // inside dev
  std::vector<LayerDev> h_layers;   // host mirror of d_layers
};

// ---------------------------------------------------------- validation --
static jolt_status validate_desc(const jolt_cache_desc *d) {
  if (!d) return fail(JOLT_E_INVALID, "desc is NULL");
  if (d->n_layers < 1 || d->n_groups < 1 || d->n_groups > d->n_layers)
    return fail(JOLT_E_INVALID, "n_layers=%d n_groups=%d", d->n_layers, d->n_groups);
  if (d->n_kv_heads < 1 || d->n_q_heads < 1 || d->n_q_heads % d->n_kv_heads)
    return fail(JOLT_E_INVALID, "n_q_heads=%d must be a positive multiple of n_kv_heads=%d",
                d->n_q_heads, d->n_kv_heads);
  if (d->head_dim < 2 || d->head_dim % 2)
    return fail(JOLT_E_INVALID, "head_dim=%d must be even", d->head_dim);
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(JOLT_E_UNSUPPORTED, "head_dim=%d: supported 64, 128", d->head_dim);
  if (d->n_q_heads / d->n_kv_heads > kMaxHg)
    return fail(JOLT_E_UNSUPPORTED, "query heads per KV head %d > %d",
                d->n_q_heads / d->n_kv_heads, kMaxHg);
  if (d->T < 1) return fail(JOLT_E_INVALID, "T=%d must be >= 1", d->T);
  if (d->T > kMaxPos) return fail(JOLT_E_UNSUPPORTED, "T=%d > %d", d->T, kMaxPos);
  if (d->factor_dtype != JOLT_F32 && d->factor_dtype != JOLT_BF16)
    return fail(JOLT_E_INVALID, "factor_dtype=%d", (int)d->factor_dtype);
  if (!d->group_start || !d->cells) return fail(JOLT_E_INVALID, "group_start or cells is NULL");
  if (d->group_start[0] != 0 || d->group_start[d->n_groups] != d->n_layers)
    return fail(JOLT_E_INVALID, "group_start must run from 0 to n_layers");
  for (int g = 0; g < d->n_groups; ++g)
    if (d->group_start[g + 1] <= d->group_start[g])
      return fail(JOLT_E_INVALID, "group_start not strictly increasing at %d", g);
  for (int g = 0; g < d->n_groups; ++g) {
    int gs = d->group_start[g + 1] - d->group_start[g];
    int64_t rmax = std::min<int64_t>(d->T, (int64_t)gs * d->n_kv_heads * d->head_dim);
    for (int tau = 0; tau < 2; ++tau) {
      const jolt_cell &c = d->cells[2 * g + tau];
      if (c.r_T < 0 || c.r_T > rmax || c.r_F < 0 || c.r_F > d->head_dim)
        return fail(JOLT_E_INVALID, "cell (%d,%d): r_T=%d (max %lld), r_F=%d (max %d)", g, tau,
                    c.r_T, (long long)rmax, c.r_F, d->head_dim);
      if ((c.r_T == 0) != (c.r_F == 0))
        return fail(JOLT_E_INVALID, "cell (%d,%d): r_T=%d and r_F=%d must be zero together", g,
                    tau, c.r_T, c.r_F);
      if (c.bits != 0 && c.bits != 2 && c.bits != 4 && c.bits != 8)
        return fail(JOLT_E_INVALID, "cell (%d,%d): bits=%d not in {0,2,4,8}", g, tau, c.bits);
      if (c.r_T > 0 && (!c.A || !c.B || !c.G))
        return fail(JOLT_E_INVALID, "cell (%d,%d): A, B, G required when r_T > 0", g, tau);
      if ((c.bits > 0) != (c.codes != nullptr) || (c.bits > 0) != (c.scales != nullptr))
        return fail(JOLT_E_INVALID, "cell (%d,%d): codes/scales must be non-NULL iff bits > 0",
                    g, tau);
    }
  }
  return JOLT_OK;
}

// ------------------------------------------------------- layout builder --
// One host staging buffer mirrors the single device allocation.
struct Staging {
  std::vector<uint8_t> buf;
  size_t take(size_t bytes) {
    size_t off = buf.size();
    buf.resize(off + align256(bytes), 0);
    return off;
  }
};

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

extern "C" jolt_status jolt_load_cache(const jolt_cache_desc *desc, jolt_stream stream,
                                       jolt_cache **out) {
  if (!out) return fail(JOLT_E_INVALID, "out is NULL");
  *out = nullptr;
  jolt_status st = validate_desc(desc);
  if (st != JOLT_OK) return st;
  const char *fa = std::getenv("JOLT_TEST_FAIL_ALLOC");
  if (fa && fa[0] == '1') return fail(JOLT_E_OOM, "allocation failure forced by JOLT_TEST_FAIL_ALLOC");

  jolt_cache *c = new (std::nothrow) jolt_cache();
  if (!c) return fail(JOLT_E_OOM, "host allocation failed");
  const int H = desc->n_kv_heads, d = desc->head_dim, T = desc->T;
  const bool f32 = desc->factor_dtype == JOLT_F32;
  const int fb = f32 ? 4 : 2;
  c->n_layers = desc->n_layers;
  c->n_groups = desc->n_groups;
  c->H = H;
  c->H_q = desc->n_q_heads;
  c->d = d;
  c->T = T;
  c->T_pad = round_up(T, kTokPad);
  c->f32 = f32;
  c->group_start.assign(desc->group_start, desc->group_start + desc->n_groups + 1);
  c->layer_group.resize(c->n_layers);
  for (int g = 0; g < c->n_groups; ++g)
    for (int l = c->group_start[g]; l < c->group_start[g + 1]; ++l) c->layer_group[l] = g;
  const int T_pad = c->T_pad;

  std::vector<double> Pi64((size_t)d * d);
  make_rotation(desc->rotation_seed, d, Pi64.data());

  Staging S;
  try {
    size_t off_pi = S.take(sizeof(float) * d * d);
    for (int i = 0; i < d * d; ++i) ((float *)(S.buf.data() + off_pi))[i] = (float)Pi64[i];
    size_t off_pit = S.take(sizeof(float) * d * d);
    for (int r = 0; r < d; ++r)
      for (int c2 = 0; c2 < d; ++c2)
        ((float *)(S.buf.data() + off_pit))[(size_t)c2 * d + r] = (float)Pi64[(size_t)r * d + c2];
    // Pi in fp16 with padded rows: the MFMA kernel copies it to LDS as it is
    const int pik_row = d + kRowPad;
    size_t off_pik = S.take(sizeof(_Float16) * d * pik_row);
    for (int r = 0; r < d; ++r)
      for (int c2 = 0; c2 < d; ++c2)
        ((_Float16 *)(S.buf.data() + off_pik))[(size_t)r * pik_row + c2] = (_Float16)Pi64[(size_t)r * d + c2];

    struct Offs {
      size_t A, B, Bt;
      std::vector<size_t> G, W2, codes, scales;  // per layer in group
    };
    std::vector<Offs> offs(2 * c->n_groups);
    c->cells.resize(2 * c->n_groups);
    for (int g = 0; g < c->n_groups; ++g) {
      const int gs = c->group_start[g + 1] - c->group_start[g];
      for (int tau = 0; tau < 2; ++tau) {
        const jolt_cell &in = desc->cells[2 * g + tau];
        CellMeta m;
        m.rT = in.r_T;
        m.rF = in.r_F;
        m.bits = in.bits;
        // ranks above 256 pad to 64, so wide key tiles take an even number of
        // 32-rank MFMA steps (fewer kernel instantiations)
        m.rT_pad = round_up(in.r_T, in.r_T > 8 * kRankPad ? 2 * kRankPad : kRankPad);
        m.rF_pad = round_up(in.r_F, kRankPad);
        c->cells[2 * g + tau] = m;
        Offs &o = offs[2 * g + tau];
        // A.  bf16 caches: fp16 scaled by a power of two a_s (exact for every
        // bf16 value in fp16's normal range) so that the MFMA products take A
        // as it is -- A_K rows in the key tile, A_V against fp16 softmax
        // weights (11-bit, where bf16 weights would carry 8); W2 carries the
        // 1 / a_s.
        o.A = S.take((size_t)fb * T_pad * std::max(m.rT_pad, 1));
        m.a_s = 1.0;
        const bool a16 = !f32;
        if (a16) {
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
            size_t dst = tau == 0 ? (size_t)t * m.rT_pad + r : av_index(t, r, m.rT_pad);
            if (a16)
              ((_Float16 *)(S.buf.data() + o.A))[dst] =
                  (_Float16)(load_factor(in.A, (size_t)t * m.rT + r, false) * (float)m.a_s);
            else
              store_factor(S.buf.data() + o.A, dst, in.A, (size_t)t * m.rT + r, f32);
          }
        c->cells[2 * g + tau].a_s = m.a_s;
        // B
        o.B = S.take((size_t)fb * d * std::max(m.rF_pad, 1));
        for (int f = 0; f < d; ++f)
          for (int j = 0; j < m.rF; ++j)
            store_factor(S.buf.data() + o.B, (size_t)f * m.rF_pad + j, in.B, (size_t)f * m.rF + j,
                         f32);
        // B^T in float32 for the value finalize
        o.Bt = S.take(sizeof(float) * std::max(m.rF_pad, 1) * d);
        for (int f = 0; f < d; ++f)
          for (int j = 0; j < m.rF; ++j)
            ((float *)(S.buf.data() + o.Bt))[(size_t)j * d + f] =
                load_factor(in.B, (size_t)f * m.rF + j, f32);
        // G and residual, per layer of the group
        for (int lp = 0; lp < gs; ++lp) {
          size_t og = S.take((size_t)fb * H * std::max(m.rT_pad, 1) * std::max(m.rF_pad, 1));
          o.G.push_back(og);
          for (int h = 0; h < H; ++h)
            for (int r = 0; r < m.rT; ++r)
              for (int j = 0; j < m.rF; ++j) {
                size_t src = (((size_t)lp * H + h) * m.rT + r) * m.rF + j;
                size_t dst = tau == 0 ? ((size_t)h * m.rF_pad + j) * m.rT_pad + r
                                      : ((size_t)h * m.rT_pad + r) * m.rF_pad + j;
                store_factor(S.buf.data() + og, dst, in.G, src, f32);
              }
          // W2[h] = B G[lp, h]^T (bf16 caches): key-tile matrix (divided by
          // a_s, the scale of the fp16 A_K) and value-finalize matrix, fp16,
          // formed in float64 and rounded once
          if (!f32 && m.rT > 0) {
            // key rows padded like their LDS image
            const int w2_row = m.rT_pad + (tau == 0 ? kRowPad : 0);
            size_t ow = S.take(sizeof(uint16_t) * H * d * w2_row);
            o.W2.push_back(ow);
            _Float16 *W2 = (_Float16 *)(S.buf.data() + ow);
            std::vector<double> Bf((size_t)d * m.rF), Gf((size_t)m.rT * m.rF);
            for (size_t i = 0; i < Bf.size(); ++i) Bf[i] = load_factor(in.B, i, false);
            for (int hh = 0; hh < H; ++hh) {
              for (size_t i = 0; i < Gf.size(); ++i)
                Gf[i] = load_factor(in.G, ((size_t)lp * H + hh) * m.rT * m.rF + i, false);
              for (int f = 0; f < d; ++f)
                for (int col = 0; col < m.rT_pad; ++col) {
                  const int r = col;
                  double acc = 0.0;
                  if (r < m.rT)
                    for (int j = 0; j < m.rF; ++j) acc += Bf[(size_t)f * m.rF + j] * Gf[(size_t)r * m.rF + j];
                  W2[((size_t)hh * d + f) * w2_row + col] = (_Float16)(acc / m.a_s);
                }
            }
          } else {
            o.W2.push_back(0);
          }
          if (m.bits == 0) {
            o.codes.push_back(0);
            o.scales.push_back(0);
            continue;
          }
          const int b = m.bits, rowb = d * b / 8;
          size_t oc = S.take((size_t)H * T_pad * rowb);
          size_t os = S.take(sizeof(float) * H * T_pad);
          o.codes.push_back(oc);
          o.scales.push_back(os);
          uint8_t *C = S.buf.data() + oc;
          float *Sc = (float *)(S.buf.data() + os);
          for (int h = 0; h < H; ++h)
            for (int t = 0; t < T; ++t) {
              const uint8_t *row = in.codes + (((size_t)lp * H + h) * T + t) * rowb;
              Sc[(size_t)h * T_pad + t] = in.scales[((size_t)lp * H + h) * T + t];
              for (int i = 0; i < d; ++i) {
                uint32_t code = (uint32_t)canon_code(row, i, b);
                int dw, sh;
                if (tau == 0) {
                  int s = i >> 5, g2 = (i >> 3) & 3, j = i & 7;
                  code_pos(8 * s + j, b, &dw, &sh);
                  uint32_t *w = (uint32_t *)(C + ((size_t)h * T_pad + t) * rowb + g2 * (d * b / 32));
                  w[dw] |= code << sh;
                } else {
                  size_t at;
                  vcode_pos(h, t, i, b, T_pad, d, &at, &sh);
                  *(uint32_t *)(C + at) |= code << sh;
                }
              }
            }
        }
      }
    }
    size_t off_layers = S.take(sizeof(LayerDev) * c->n_layers);
    c->dev_bytes = S.buf.size();
    hipError_t e = hipMalloc(&c->dev, c->dev_bytes);
    if (e != hipSuccess) {
      delete c;
      return fail(e == hipErrorOutOfMemory ? JOLT_E_OOM : JOLT_E_HIP, "hipMalloc(%zu): %s",
                  S.buf.size(), hipGetErrorString(e));
    }
    hipGetDevice(&c->device);
    uint8_t *base = (uint8_t *)c->dev;
    c->h_layers.resize(c->n_layers);
    for (int l = 0; l < c->n_layers; ++l) {
      const int g = c->layer_group[l], lp = l - c->group_start[g];
      LayerDev &L = c->h_layers[l];
      std::memset(&L, 0, sizeof L);
      L.Pi = (const float *)(base + off_pi);
      L.PiT = (const float *)(base + off_pit);
      L.PiK = (const _Float16 *)(base + off_pik);
      L.T = T;
      L.T_pad = T_pad;
      L.f32 = f32 ? 1 : 0;
      for (int tau = 0; tau < 2; ++tau) {
        const CellMeta &m = c->cells[2 * g + tau];
        const Offs &o = offs[2 * g + tau];
        CellDev &cd = L.c[tau];
        cd.A = base + o.A;
        cd.B = base + o.B;
        cd.Bt = (const float *)(base + o.Bt);
        cd.G = base + o.G[lp];
        cd.W2 = o.W2[lp] ? (const void *)(base + o.W2[lp]) : nullptr;
        cd.codes = m.bits ? base + o.codes[lp] : nullptr;
        cd.scales = m.bits ? (const float *)(base + o.scales[lp]) : nullptr;
        cd.rT = m.rT;
        cd.rF = m.rF;
        cd.bits = m.bits;
        cd.rT_pad = m.rT_pad;
        cd.rF_pad = m.rF_pad;
        cd.a_inv = (float)(1.0 / m.a_s);
      }
    }
    std::memcpy(S.buf.data() + off_layers, c->h_layers.data(), sizeof(LayerDev) * c->n_layers);
    c->d_layers = (LayerDev *)(base + off_layers);
    hipStream_t s = (hipStream_t)stream;
    e = hipMemcpyAsync(c->dev, S.buf.data(), S.buf.size(), hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) {
      hipFree(c->dev);
      delete c;
      return fail(JOLT_E_HIP, "upload: %s", hipGetErrorString(e));
    }
  } catch (const std::bad_alloc &) {
    if (c->dev) hipFree(c->dev);
    delete c;
    return fail(JOLT_E_OOM, "host staging allocation failed");
  }
  *out = c;
  return ok();
}

extern "C" jolt_status jolt_free_cache(jolt_cache *c) {
  if (!c) return ok();
  hipError_t e = c->dev ? hipFree(c->dev) : hipSuccess;
  delete c;
  if (e != hipSuccess) return fail(JOLT_E_HIP, "hipFree: %s", hipGetErrorString(e));
  return ok();
}

extern "C" jolt_status jolt_cache_info(const jolt_cache *c, int32_t *n_layers, int32_t *n_kv,
                                       int32_t *n_q, int32_t *d, int32_t *T, size_t *bytes) {
  if (!c) return fail(JOLT_E_INVALID, "cache is NULL");
  if (n_layers) *n_layers = c->n_layers;
  if (n_kv) *n_kv = c->H;
  if (n_q) *n_q = c->H_q;
  if (d) *d = c->d;
  if (T) *T = c->T;
  if (bytes) *bytes = c->dev_bytes;
  return ok();
}

// ------------------------------------------------------- decode planning --
struct Plan {
  int kernel;        // JOLT_KERNEL_GENERIC or JOLT_KERNEL_MFMA
  int split_tokens, n_split, rV_max, stride, T_max;
  size_t ws_bytes;
};

// The MFMA kernel stages W2_K[h] = B_K G_K[h]^T / s and (with a key
// residual) Pi in LDS as fp16 rows padded by 8 elements, next to 1 KiB of
// per-wave softmax state, 8 KiB of rotated queries, the RoPE frequencies,
// 4 KiB of query MFMA operands and the fp32 sums of the waves' value
// partials (1 KiB per 16 value ranks, 8 KiB for the residual); after the
// tile loop the W2_K / Pi region holds every wave's fp16 value partial;
// key ranks up to 256 are prefetched a tile ahead in registers and value
// ranks up to 512 accumulate in registers.
// hg1: one query per KV head.  The classes launched as HG1 variants (value
// ranks above 128, or key ranks above 256) park 4 lanes' worth of each value
// block per wave instead of 64, and with key ranks up to 256 run 8 waves.
static int mfma_lds_bytes(const CellDev &k, const CellDev &v, int d, bool hg1) {
  // key ranks above 256 keep Pi in registers (4 waves), not in LDS
  const bool wide = k.rT_pad > 8 * kRankPad;
  const int kpath = 2 * d * (k.rT_pad + kRowPad) + (k.bits > 0 && !wide ? 2 * d * (d + kRowPad) : 0);
  const bool big_v = v.rT_pad / 16 > 8;
  const bool hg1v = hg1 && (wide || big_v);  // launched as an HG1 variant
  const int waves = wide || (big_v && !hg1v) ? 4 : 8;
  // fp16 value partials of every wave
  const int park = waves * (v.rT_pad / 16 + 8) * (hg1v ? 32 : 512);
  // + softmax reduction, frequencies (and / 2 pi), query operands, combined
  // value tiles and the token-block counter
  return std::max(kpath, park) + 1024 + 512 + 6144 + 1024 * (v.rT_pad / 16 + 8) + 16;
}

static bool mfma_ok(const jolt_cache *c, int layer, int *lds) {
  if (c->f32 || c->d != 128) return false;
  const LayerDev &L = c->h_layers[layer];
  const CellDev &k = L.c[0], &v = L.c[1];
  if (v.rT_pad > 512 || k.rT_pad > 512) return false;
  if (k.rT_pad > 8 * kRankPad && v.rT_pad > 256) return false;  // no such class
  *lds = mfma_lds_bytes(k, v, c->d, c->H_q == c->H);
  return *lds <= jolt_mfma_max_lds();
}

// Two sequences share one MFMA launch when their layer's key bits, value
// bits and padded key rank match.
static bool same_class(const jolt_cache *a, const jolt_cache *b, int layer) {
  const CellDev &ka = a->h_layers[layer].c[0], &va = a->h_layers[layer].c[1];
  const CellDev &kb = b->h_layers[layer].c[0], &vb = b->h_layers[layer].c[1];
  return ka.bits == kb.bits && va.bits == vb.bits && ka.rT_pad == kb.rT_pad;
}

// Compute units of the current device (cached per device).
static int cu_count() {
  static int cached[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cached[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

static jolt_status plan_decode(const jolt_cache *const *caches, int batch, int layer,
                               const jolt_launch *launch, Plan *p) {
  if (batch < 0) return fail(JOLT_E_INVALID, "batch=%d", batch);
  if (batch > 0 && !caches) return fail(JOLT_E_INVALID, "caches is NULL");
  const jolt_cache *c0 = batch ? caches[0] : nullptr;
  for (int b = 0; b < batch; ++b) {
    const jolt_cache *c = caches[b];
    if (!c) return fail(JOLT_E_INVALID, "caches[%d] is NULL", b);
    if (c->n_layers != c0->n_layers || c->H != c0->H || c->H_q != c0->H_q || c->d != c0->d ||
        c->group_start != c0->group_start || c->f32 != c0->f32)
      return fail(JOLT_E_INVALID,
                  "caches[%d] differs in layers, groups, heads, head_dim or factor dtype", b);
  }
  if (batch && (layer < 0 || layer >= c0->n_layers))
    return fail(JOLT_E_INVALID, "layer=%d out of range [0,%d)", layer, c0->n_layers);
  int want = launch ? launch->kernel : JOLT_KERNEL_AUTO;
  if (want < 0 || want > 2) return fail(JOLT_E_INVALID, "launch->kernel=%d", want);
  if (launch && launch->split_tokens < 0)
    return fail(JOLT_E_INVALID, "launch->split_tokens=%d", launch->split_tokens);
  p->T_max = 1;
  p->rV_max = 0;
  bool mf = batch > 0;
  for (int b = 0; b < batch; ++b) {
    const jolt_cache *c = caches[b];
    p->T_max = std::max(p->T_max, c->T);
    p->rV_max = std::max(p->rV_max, c->h_layers[layer].c[1].rT_pad);
    int lds = 0;
    if (!mfma_ok(c, layer, &lds)) mf = false;
  }
  if (want == JOLT_KERNEL_MFMA && !mf)
    return fail(JOLT_E_UNSUPPORTED,
                "MFMA kernel needs bf16 factors, d=128, key rank <= 512, value rank <= 512 (<= 256 "
                "with key ranks above 256) and an LDS fit for W2_K and Pi");
  p->kernel = (want == JOLT_KERNEL_GENERIC || !mf) ? JOLT_KERNEL_GENERIC : JOLT_KERNEL_MFMA;
  const int tile = p->kernel == JOLT_KERNEL_MFMA ? kTokPad : 32;
  int H = batch ? c0->H : 1;
  int split = launch && launch->split_tokens > 0 ? launch->split_tokens : 0;
  if (split == 0) {
    // one workgroup per compute unit: the MFMA kernel holds a CU alone
    // (LDS and registers), and fewer, longer splits pay the per-workgroup
    // prologue and epilogue less often.  The MFMA kernel runs one launch per
    // (key bits, value bits, key-rank steps) class of the batch, one after
    // the other, so the split count is sized for the smallest class (a
    // one-sequence class would otherwise fill a fraction of the CUs) and
    // capped at about four rounds of workgroups for the largest.
    int want_wg = p->kernel == JOLT_KERNEL_MFMA ? cu_count() : 512;
    int units = batch;
    if (p->kernel == JOLT_KERNEL_MFMA && batch > 1) {
      int cmin = batch, cmax = 1;
      for (int i = 0; i < batch; ++i) {
        int n = 0;
        for (int j = 0; j < batch; ++j) n += same_class(caches[j], caches[i], layer);
        cmin = std::min(cmin, n);
        cmax = std::max(cmax, n);
      }
      units = std::max(cmin, (cmax + 3) / 4);
    }
    int n = std::max(1, (want_wg + units * H - 1) / std::max(1, units * H));
    split = (p->T_max + n - 1) / n;
  }
  p->split_tokens = round_up(std::max(split, 1), tile);
  p->split_tokens = std::max(p->split_tokens, round_up((p->T_max + kMaxSplits - 1) / kMaxSplits, tile));
  p->n_split = (p->T_max + p->split_tokens - 1) / p->split_tokens;
  p->stride = p->kernel == JOLT_KERNEL_MFMA ? 4 + (batch ? c0->d : 0)
                                            : partial_stride(p->rV_max, batch ? c0->d : 0);
  p->ws_bytes = (size_t)batch * (batch ? c0->H_q : 0) * p->n_split * p->stride * sizeof(float);
  return JOLT_OK;
}

extern "C" jolt_status jolt_decode_workspace_size(const jolt_cache *const *caches, int32_t batch,
                                                  int32_t layer, const jolt_launch *launch,
                                                  size_t *bytes) {
  if (!bytes) return fail(JOLT_E_INVALID, "bytes is NULL");
  Plan p;
  jolt_status st = plan_decode(caches, batch, layer, launch, &p);
  if (st != JOLT_OK) return st;
  *bytes = p.ws_bytes;
  return ok();
}

extern "C" jolt_status jolt_decode_attention(const jolt_cache *const *caches, int32_t batch,
                                             int32_t layer, const void *q, jolt_dtype q_dtype,
                                             const int32_t *q_pos, const float *inv_freq,
                                             float softmax_scale, float *out, void *workspace,
                                             size_t ws_bytes, const jolt_launch *launch,
                                             jolt_stream stream) {
  Plan p;
  jolt_status st = plan_decode(caches, batch, layer, launch, &p);
  if (st != JOLT_OK) return st;
  if (batch == 0) return ok();
  if (!q || !q_pos || !inv_freq || !out) return fail(JOLT_E_INVALID, "NULL q/q_pos/inv_freq/out");
  if (q_dtype != JOLT_F32 && q_dtype != JOLT_BF16) return fail(JOLT_E_INVALID, "q_dtype");
  if (!std::isfinite(softmax_scale)) return fail(JOLT_E_INVALID, "softmax_scale not finite");
  if (check_rope(q_pos, batch, inv_freq, caches[0]->d) != JOLT_OK)
    return fail(JOLT_E_INVALID, "q_pos must lie in [0, 2^20] and inv_freq in [0, 1]");
  if (!workspace || ws_bytes < p.ws_bytes)
    return fail(JOLT_E_WORKSPACE, "workspace %zu bytes, need %zu", workspace ? ws_bytes : 0,
                p.ws_bytes);
  const jolt_cache *c0 = caches[0];
  hipStream_t s = (hipStream_t)stream;
  DecodeArgs a;
  std::memset(&a, 0, sizeof a);
  a.scale = softmax_scale;
  a.q_f32 = q_dtype == JOLT_F32;
  a.f32 = c0->f32 ? 1 : 0;
  a.H = c0->H;
  a.H_q = c0->H_q;
  a.Hg = c0->H_q / c0->H;
  a.d = c0->d;
  for (int i = 0; i < c0->d / 2; ++i) a.inv_freq[i] = inv_freq[i];
  a.n_split = p.n_split;
  a.split_tokens = p.split_tokens;
  a.stride = p.stride;
  a.rV_max = p.rV_max;
  const size_t qbytes = (size_t)c0->H_q * c0->d * (a.q_f32 ? 4 : 2);
  for (int b0 = 0; b0 < batch; b0 += kMaxBatchPerLaunch) {
    int nb = std::min(kMaxBatchPerLaunch, batch - b0);
    a.q = (const uint8_t *)q + b0 * qbytes;
    a.out = out + (size_t)b0 * c0->H_q * c0->d;
    a.ws = (float *)workspace + (size_t)b0 * c0->H_q * p.n_split * p.stride;
    hipError_t e = hipSuccess;
    // timing events: the first split launch's start and the last one's end
    KernelEvents ev;
    if (launch && b0 == 0) ev.begin = (hipEvent_t)launch->ev_begin;
    hipEvent_t ev_last = launch && b0 + nb >= batch ? (hipEvent_t)launch->ev_end : nullptr;
    if (p.kernel == JOLT_KERNEL_MFMA) {
      // one launch per (key bits, value bits, key-rank steps) class of the
      // chunk's sequences; every launch writes its sequences' rows of the
      // chunk's workspace
      MfmaArgs ma;
      std::memset(&ma, 0, sizeof ma);
      ma.q = a.q;
      ma.ws = a.ws;
      std::memcpy(ma.inv_freq, a.inv_freq, sizeof ma.inv_freq);
      ma.scale = a.scale;
      ma.q_f32 = a.q_f32;
      ma.H = a.H;
      ma.H_q = a.H_q;
      ma.Hg = a.Hg;
      ma.n_split = a.n_split;
      ma.split_tokens = a.split_tokens;
      ma.stride = a.stride;
      ma.grid8 = (a.n_split & 7) == 0;
      bool done[kMaxBatchPerLaunch] = {};
      int last_class = 0;  // first member of the chunk's last launch class
      for (int i0 = 0; i0 < nb; ++i0) {
        bool first = true;
        for (int i = 0; i < i0 && first; ++i) first = !same_class(caches[b0 + i], caches[b0 + i0], layer);
        if (first) last_class = i0;
      }
      for (int i0 = 0; i0 < nb; ++i0) {
        if (done[i0]) continue;
        const CellDev &k0 = caches[b0 + i0]->h_layers[layer].c[0];
        const CellDev &v0 = caches[b0 + i0]->h_layers[layer].c[1];
        int n = 0, nkt = 0, rv = 0, lds = 0;
        for (int i = i0; i < nb; ++i) {
          const jolt_cache *c = caches[b0 + i];
          const CellDev &k = c->h_layers[layer].c[0], &v = c->h_layers[layer].c[1];
          if (done[i] || !same_class(c, caches[b0 + i0], layer)) continue;
          done[i] = true;
          const LayerDev &L = c->h_layers[layer];
          SeqMfma &m = ma.seq[n];
          m.kA = k.A;
          m.kcodes = k.codes;
          m.kW2 = k.W2;
          m.kscales = k.scales;
          m.vA = v.A;
          m.vcodes = v.codes;
          m.vW2 = v.W2;
          m.vscales = v.scales;
          m.PiK = L.PiK;
          m.T = c->T;
          m.T_pad = L.T_pad;
          m.q_pos = q_pos[b0 + i];
          m.slot = i;
          m.vrT_pad = v.rT_pad;
          ++n;
          nkt = k.rT_pad / kRankPad;
          rv = std::max(rv, v.rT_pad);
          lds = std::max(lds, mfma_lds_bytes(k, v, c->d, c->H_q == c->H));
        }
        ma.nseq = n;
        ma.rV_max = rv;
        // frequency blocks of 16 whose angles stay below kRopeSmall for every
        // cached position of the launch's sequences
        int t_max = 0;
        for (int i = 0; i < n; ++i) t_max = std::max(t_max, ma.seq[i].T);
        ma.rope_small = 0;
        for (int m = 0; m < c0->d / 32; ++m) {
          double w = 0.0;
          for (int f = 16 * m; f < 16 * m + 16; ++f) w = std::max(w, (double)inv_freq[f]);
          if (w * (double)std::max(t_max - 1, 0) <= kRopeSmall) ma.rope_small |= 1 << m;
        }
        if (i0 == last_class) ev.end = ev_last;
        e = jolt_launch_mfma(ma, n, k0.bits, v0.bits, nkt, lds, s, ev);
        if (e != hipSuccess) return fail(JOLT_E_HIP, "split kernel launch: %s", hipGetErrorString(e));
        ev.begin = nullptr;
      }
    } else {
      a.nseq = nb;
      for (int i = 0; i < nb; ++i) {
        a.seq[i].layer = caches[b0 + i]->d_layers + layer;
        a.seq[i].q_pos = q_pos[b0 + i];
        a.seq[i].T = caches[b0 + i]->T;
        a.seq[i].slot = i;
      }
      ev.end = ev_last;
      e = jolt_launch_generic(a, nb, s, ev);
      if (e != hipSuccess) return fail(JOLT_E_HIP, "split kernel launch: %s", hipGetErrorString(e));
    }
    a.nseq = nb;
    e = p.kernel == JOLT_KERNEL_MFMA ? jolt_launch_merge_outputs(a, nb, s) : jolt_launch_merge(a, nb, s);
    if (e != hipSuccess) return fail(JOLT_E_HIP, "merge kernel launch: %s", hipGetErrorString(e));
  }
  return ok();
}

// ----------------------------------------------------------------- dense --
static jolt_status plan_dense(int batch, int n_kv, int n_q, int d, int T, const jolt_launch *launch,
                              int *split_tokens, int *n_split, size_t *bytes) {
  if (batch < 0 || n_kv < 1 || n_q < 1 || T < 1 || n_q % n_kv)
    return fail(JOLT_E_INVALID, "batch=%d n_kv=%d n_q=%d T=%d", batch, n_kv, n_q, T);
  if (d != 64 && d != 128) return fail(JOLT_E_UNSUPPORTED, "d=%d: supported 64, 128", d);
  if (n_q / n_kv > kMaxHg) return fail(JOLT_E_UNSUPPORTED, "n_q/n_kv > %d", kMaxHg);
  if (launch && launch->split_tokens < 0) return fail(JOLT_E_INVALID, "split_tokens < 0");
  int split = launch && launch->split_tokens > 0 ? launch->split_tokens : 0;
  if (split == 0) {
    int n = std::max(1, (1024 + batch * n_kv - 1) / std::max(1, batch * n_kv));
    split = (T + n - 1) / n;
  }
  *split_tokens = round_up(std::max(split, 1), 64);
  *split_tokens = std::max(*split_tokens, round_up((T + kMaxSplits - 1) / kMaxSplits, 64));
  *n_split = (T + *split_tokens - 1) / *split_tokens;
  *bytes = (size_t)batch * n_q * *n_split * (4 + d) * sizeof(float);
  return JOLT_OK;
}

extern "C" jolt_status jolt_dense_workspace_size(int32_t batch, int32_t n_kv, int32_t n_q,
                                                 int32_t d, int32_t T, const jolt_launch *launch,
                                                 size_t *bytes) {
  if (!bytes) return fail(JOLT_E_INVALID, "bytes is NULL");
  int st_, ns;
  jolt_status st = plan_dense(batch, n_kv, n_q, d, T, launch, &st_, &ns, bytes);
  return st == JOLT_OK ? ok() : st;
}

extern "C" jolt_status jolt_dense_attention(const void *k_rope, const void *v, jolt_dtype kv_dtype,
                                            int32_t batch, int32_t n_kv, int32_t n_q, int32_t d,
                                            int32_t T, const void *q, jolt_dtype q_dtype,
                                            const int32_t *q_pos, const float *inv_freq,
                                            float softmax_scale, float *out, void *workspace,
                                            size_t ws_bytes, const jolt_launch *launch,
                                            jolt_stream stream) {
  int split_tokens, n_split;
  size_t need;
  jolt_status st = plan_dense(batch, n_kv, n_q, d, T, launch, &split_tokens, &n_split, &need);
  if (st != JOLT_OK) return st;
  if (batch == 0) return ok();
  if (!k_rope || !v || !q || !q_pos || !inv_freq || !out)
    return fail(JOLT_E_INVALID, "NULL pointer argument");
  if ((kv_dtype != JOLT_F32 && kv_dtype != JOLT_BF16) || (q_dtype != JOLT_F32 && q_dtype != JOLT_BF16))
    return fail(JOLT_E_INVALID, "dtype");
  if (!std::isfinite(softmax_scale)) return fail(JOLT_E_INVALID, "softmax_scale not finite");
  if (check_rope(q_pos, batch, inv_freq, d) != JOLT_OK)
    return fail(JOLT_E_INVALID, "q_pos must lie in [0, 2^20] and inv_freq in [0, 1]");
  if (T > kMaxPos) return fail(JOLT_E_UNSUPPORTED, "T=%d > %d", T, kMaxPos);
  if (!workspace || ws_bytes < need)
    return fail(JOLT_E_WORKSPACE, "workspace %zu bytes, need %zu", workspace ? ws_bytes : 0, need);
  DenseArgs a;
  std::memset(&a, 0, sizeof a);
  a.scale = softmax_scale;
  a.kv_f32 = kv_dtype == JOLT_F32;
  a.q_f32 = q_dtype == JOLT_F32;
  a.H = n_kv;
  a.H_q = n_q;
  a.Hg = n_q / n_kv;
  a.d = d;
  a.T = T;
  a.n_split = n_split;
  a.split_tokens = split_tokens;
  for (int i = 0; i < d / 2; ++i) a.inv_freq[i] = inv_freq[i];
  const size_t kvb = (size_t)n_kv * T * d * (a.kv_f32 ? 4 : 2);
  const size_t qb = (size_t)n_q * d * (a.q_f32 ? 4 : 2);
  hipStream_t s = (hipStream_t)stream;
  for (int b0 = 0; b0 < batch; b0 += kMaxBatchPerLaunch) {
    int nb = std::min(kMaxBatchPerLaunch, batch - b0);
    a.k = (const uint8_t *)k_rope + b0 * kvb;
    a.v = (const uint8_t *)v + b0 * kvb;
    a.q = (const uint8_t *)q + b0 * qb;
    a.out = out + (size_t)b0 * n_q * d;
    a.ws = (float *)workspace + (size_t)b0 * n_q * n_split * (4 + d);
    a.batch = nb;
    a.seq0 = b0;
    for (int i = 0; i < nb; ++i) a.q_pos[i] = q_pos[b0 + i];
    hipError_t e = jolt_launch_dense(a, nb, s);
    if (e != hipSuccess) return fail(JOLT_E_HIP, "dense launch: %s", hipGetErrorString(e));
    e = jolt_launch_dense_merge(a, nb, s);
    if (e != hipSuccess) return fail(JOLT_E_HIP, "dense merge launch: %s", hipGetErrorString(e));
  }
  return ok();
}

// --------------------------------------------------------- test helpers --
extern "C" jolt_status jolt_make_rotation(uint64_t seed, int32_t d, double *out) {
  if (!out || d < 1 || d > 4096) return fail(JOLT_E_INVALID, "out NULL or d=%d", d);
  jolt::make_rotation(seed, d, out);
  return ok();
}

extern "C" jolt_status jolt_debug_unpack(const jolt_cache *c, int32_t layer, int32_t tau,
                                         uint8_t *codes_out, jolt_stream stream) {
  if (!c || !codes_out) return fail(JOLT_E_INVALID, "NULL argument");
  if (layer < 0 || layer >= c->n_layers || (tau != 0 && tau != 1))
    return fail(JOLT_E_INVALID, "layer=%d tau=%d", layer, tau);
  if (c->h_layers[layer].c[tau].bits == 0) return fail(JOLT_E_INVALID, "cell has bits == 0");
  hipStream_t s = (hipStream_t)stream;
  size_t n = (size_t)c->H * c->T * c->d;
  uint8_t *dbuf = nullptr;
  HIP_TRY(hipMalloc(&dbuf, n));
  hipError_t e = jolt_launch_unpack(c->d_layers + layer, tau, c->H, c->T, c->d, dbuf, s);
  if (e == hipSuccess) e = hipMemcpyAsync(codes_out, dbuf, n, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  hipFree(dbuf);
  if (e != hipSuccess) return fail(JOLT_E_HIP, "debug unpack: %s", hipGetErrorString(e));
  return ok();
}

extern "C" jolt_status jolt_debug_sincos(const float *angles, int32_t n, float *sin_out,
                                         float *cos_out, int32_t variant) {
  if (n < 0 || (n > 0 && (!angles || !sin_out || !cos_out)))
    return fail(JOLT_E_INVALID, "NULL argument or n < 0");
  if (variant != 0 && variant != 1) return fail(JOLT_E_INVALID, "variant %d not 0 or 1", variant);
  for (int i = 0; i < n; ++i)
    if (!(std::fabs(angles[i]) < (float)kMaxPos))
      return fail(JOLT_E_INVALID, "angle %g outside (-2^20, 2^20)", (double)angles[i]);
  if (n == 0) return ok();
  float *d = nullptr;
  HIP_TRY(hipMalloc(&d, sizeof(float) * 3 * (size_t)n));
  hipError_t e = hipMemcpy(d, angles, sizeof(float) * n, hipMemcpyHostToDevice);
  if (e == hipSuccess) e = jolt_launch_sincos(d, n, d + n, d + 2 * (size_t)n, variant, nullptr);
  if (e == hipSuccess) e = hipMemcpy(sin_out, d + n, sizeof(float) * n, hipMemcpyDeviceToHost);
  if (e == hipSuccess) e = hipMemcpy(cos_out, d + 2 * (size_t)n, sizeof(float) * n, hipMemcpyDeviceToHost);
  hipFree(d);
  if (e != hipSuccess) return fail(JOLT_E_HIP, "debug sincos: %s", hipGetErrorString(e));
  return ok();
}
