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
#include <mutex>
#include <string>
#include <vector>

#include "jolt.h"
#include "errors.h"
#include "jolt_internal.h"

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
// The same for the other translation units of the library (JOLT_OK clears
// the message).
namespace jolt {
jolt_status set_error(jolt_status st, const char *fmt, ...) {
  if (st == JOLT_OK) return ok();
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}
}  // namespace jolt

#define HIP_TRY(expr)                                                               \
  do {                                                                              \
    hipError_t e_ = (expr);                                                         \
    if (e_ != hipSuccess) return fail(JOLT_E_HIP, "%s: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

extern "C" const char *jolt_last_error(void) { return g_err.c_str(); }

// ------------------------------------------------------------- helpers --
static inline int round_up(int x, int m) { return (x + m - 1) / m * m; }

// --------------------------------------------------------- cache handle --
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

  Staged S;
  try {
    // host image of the device layout (layout.cpp): Pi from the seed, the
    // factors, W2 = B G^T and the re-packed codes
    stage_cache(desc, &S);
    c->cells = S.cells;
    const std::vector<CellOffsets> &offs = S.offs;
    size_t off_layers = S.take(sizeof(LayerDev) * c->n_layers);
    c->dev_bytes = S.buf.size();
    hipError_t e = hipMalloc(&c->dev, c->dev_bytes);
    if (e != hipSuccess) {
      delete c;
      return fail(e == hipErrorOutOfMemory ? JOLT_E_OOM : JOLT_E_HIP, "hipMalloc(%zu): %s",
                  S.buf.size(), hipGetErrorString(e));
    }
    (void)hipGetDevice(&c->device);
    uint8_t *base = (uint8_t *)c->dev;
    c->h_layers.resize(c->n_layers);
    for (int l = 0; l < c->n_layers; ++l) {
      const int g = c->layer_group[l], lp = l - c->group_start[g];
      LayerDev &L = c->h_layers[l];
      std::memset(&L, 0, sizeof L);
      L.Pi = (const float *)(base + S.off_pi);
      L.PiT = (const float *)(base + S.off_pit);
      L.PiK = (const _Float16 *)(base + S.off_pik);
      L.T = T;
      L.T_pad = T_pad;
      L.f32 = f32 ? 1 : 0;
      for (int tau = 0; tau < 2; ++tau) {
        const CellMeta &m = c->cells[2 * g + tau];
        const CellOffsets &o = offs[2 * g + tau];
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
      (void)hipFree(c->dev);
      delete c;
      return fail(JOLT_E_HIP, "upload: %s", hipGetErrorString(e));
    }
  } catch (const std::bad_alloc &) {
    if (c->dev) (void)hipFree(c->dev);
    delete c;
    return fail(JOLT_E_OOM, "host staging allocation failed");
  } catch (const std::exception &e) {
    if (c->dev) (void)hipFree(c->dev);
    delete c;
    return fail(JOLT_E_INVALID, "host staging: %s", e.what());
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
  // uncompressed tail: splits of tail_split tokens over tail_cap rows; the
  // MFMA path keeps their partials in the same rows as the split kernel's
  // (splits n_split .. n_split + n_tsplit - 1), the float32 path in a region
  // of its own at byte tail_off of the workspace
  int tail_split, n_tsplit;
  size_t tail_off;
  // one query per KV head with value ranks above 128 (key ranks up to 256):
  // the value factors in a second pass over all heads (value2.hip), with the
  // logits [batch][sc_stride / 16][H][16] at sc_off, the merge's (max, sum) at st_off
  // and the partial factor sums [batch][n2split][H][rV_max] at p2_off
  bool v2;
  int sc_stride, n2split, split2;
  size_t sc_off, st_off, p2_off;
  size_t ws_bytes;
};

// A launch class that takes the second value pass: one query per KV head
// and a value factor, with key ranks up to 256 and value ranks above 128
// (the 8-wave variant), or key ranks above 256 where W2_K and Pi fit in the
// LDS at 8 waves.  (At 4 waves the wide classes measured slower with it:
// their split kernel did not get faster without the value factors.)
static bool v2_class(int bK, int bV, int nkt, int nmv, bool hg1) {
  if (!hg1 || nmv == 0) return false;
  return nkt <= 8 ? nmv > 8 && hg1_variant(bK, bV, nkt, 9) : wide_sco(bK, nkt);
}

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
// The size is taken per sequence, with the waves and variant its own ranks
// select; a launch class that runs a sequence with fewer waves or as the
// HG1 variant (a batch mixing value ranks) uses no more LDS for it.
static int mfma_lds_bytes(const CellDev &k, const CellDev &v, int d, bool hg1) {
  // key ranks above 256 keep Pi in registers (4 waves), not in LDS
  const bool wide = k.rT_pad > 8 * kRankPad;
  const bool pi_lds = k.bits > 0 && !wide;
  const bool big_v = v.rT_pad / 16 > 8;
  // launched as an HG1 variant
  const bool hg1v = hg1 && hg1_variant(k.bits, v.bits, k.rT_pad / kRankPad, v.rT_pad / 16);
  const int waves = wide || (big_v && !hg1v) ? 4 : 8;
  return (int)mfma_lds_layout(d, k.rT_pad / kRankPad, pi_lds, v.rT_pad / 16, waves, hg1v).total;
}

static bool mfma_ok(const jolt_cache *c, int layer, int *lds) {
  if (c->f32 || c->d != 128) return false;
  const LayerDev &L = c->h_layers[layer];
  const CellDev &k = L.c[0], &v = L.c[1];
  if (v.rT_pad > 512 || k.rT_pad > 512) return false;
  if (k.rT_pad > 8 * kRankPad && v.rT_pad > 256) return false;  // no such class
  // key ranks above 256 with value ranks above 128 run on MFMA only with one
  // query per KV head (the grouped-query variant would need more registers
  // than a SIMD has; see mfma_launch.inc)
  if (k.rT_pad > 8 * kRankPad && v.rT_pad > 128 && c->H_q != c->H) return false;
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
                               const jolt_launch *launch, int tail_cap, Plan *p,
                               bool allow_v2 = true) {
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
  if (launch && launch->deterministic != 0 && launch->deterministic != 1)
    return fail(JOLT_E_INVALID, "launch->deterministic=%d", launch->deterministic);
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
  // tail splits: about one workgroup round over the batch's KV heads
  p->tail_split = p->n_tsplit = 0;
  if (tail_cap > 0) {
    const int n = std::max(1, (cu_count() + batch * H - 1) / std::max(1, batch * H));
    int ts = round_up(std::max(1, (tail_cap + n - 1) / n), 64);
    ts = std::max(ts, round_up((tail_cap + kMaxTailSplits - 1) / kMaxTailSplits, 64));
    p->tail_split = ts;
    p->n_tsplit = (tail_cap + ts - 1) / ts;
  }
  const size_t rows = (size_t)batch * (batch ? c0->H_q : 0);
  const int dd = batch ? c0->d : 0;
  if (p->kernel == JOLT_KERNEL_MFMA) {
    p->tail_off = 0;
    p->ws_bytes = rows * (p->n_split + p->n_tsplit) * p->stride * sizeof(float);
  } else {
    p->tail_off = rows * p->n_split * p->stride * sizeof(float);
    p->ws_bytes = p->tail_off + rows * p->n_tsplit * (4 + dd) * sizeof(float);
  }
  // the second value pass, if a class of the call takes it
  p->v2 = false;
  p->sc_stride = p->n2split = p->split2 = 0;
  p->sc_off = p->st_off = p->p2_off = 0;
  if (allow_v2 && p->kernel == JOLT_KERNEL_MFMA && batch > 0 && c0->H == c0->H_q && c0->H <= 32) {
    int t_pad = 0;
    for (int b = 0; b < batch; ++b) {
      const CellDev &k = caches[b]->h_layers[layer].c[0], &v = caches[b]->h_layers[layer].c[1];
      if (v2_class(k.bits, v.bits, k.rT_pad / kRankPad, v.rT_pad / 16, true)) p->v2 = true;
      t_pad = std::max(t_pad, caches[b]->h_layers[layer].T_pad);
    }
    if (p->v2) {
      auto align = [](size_t x) { return (x + 255) / 256 * 256; };
      const int H = c0->H, nb = std::min(batch, kMaxBatchPerLaunch);
      // about one workgroup per compute unit over a chunk's sequences
      const int want = std::max(1, (cu_count() + nb - 1) / nb);
      p->split2 = round_up((p->T_max + want - 1) / want, 16);
      p->n2split = (p->T_max + p->split2 - 1) / p->split2;
      p->sc_stride = t_pad;
      p->sc_off = align(p->ws_bytes);
      p->st_off = align(p->sc_off + (size_t)batch * H * t_pad * sizeof(float));
      p->p2_off = align(p->st_off + (size_t)batch * H * 2 * sizeof(float));
      p->ws_bytes = p->p2_off + (size_t)batch * p->n2split * H * p->rV_max * sizeof(float);
    }
  }
  return JOLT_OK;
}

extern "C" jolt_status jolt_decode_workspace_size(const jolt_cache *const *caches, int32_t batch,
                                                  int32_t layer, const jolt_launch *launch,
                                                  size_t *bytes) {
  if (!bytes) return fail(JOLT_E_INVALID, "bytes is NULL");
  Plan p;
  jolt_status st = plan_decode(caches, batch, layer, launch, 0, &p);
  if (st != JOLT_OK) return st;
  *bytes = p.ws_bytes;
  return ok();
}

extern "C" jolt_status jolt_decode_tail_workspace_size(const jolt_cache *const *caches,
                                                       int32_t batch, int32_t layer,
                                                       int32_t tail_cap,
                                                       const jolt_launch *launch, size_t *bytes) {
  if (!bytes) return fail(JOLT_E_INVALID, "bytes is NULL");
  if (tail_cap < 0 || tail_cap > kMaxPos) return fail(JOLT_E_INVALID, "tail_cap=%d", tail_cap);
  Plan p;
  jolt_status st = plan_decode(caches, batch, layer, launch, tail_cap, &p);
  if (st != JOLT_OK) return st;
  *bytes = p.ws_bytes;
  return ok();
}

// An uncompressed tail of post-RoPE keys and values (see jolt.h).
struct TailIn {
  const void *k = nullptr, *v = nullptr;
  jolt_dtype dtype = JOLT_BF16;
  int cap = 0;
  const int32_t *len = nullptr;
};

static jolt_status decode_impl(const jolt_cache *const *caches, int32_t batch, int32_t layer,
                               const void *q, jolt_dtype q_dtype, const int32_t *q_pos,
                               const float *inv_freq, float softmax_scale, const TailIn &tail,
                               float *out, void *workspace, size_t ws_bytes,
                               const jolt_launch *launch, jolt_stream stream,
                               bool allow_v2 = true) {
  Plan p;
  jolt_status st = plan_decode(caches, batch, layer, launch, tail.cap, &p, allow_v2);
  if (st != JOLT_OK) return st;
  if (batch == 0) return ok();
  if (!q || !q_pos || !inv_freq || !out) return fail(JOLT_E_INVALID, "NULL q/q_pos/inv_freq/out");
  if (q_dtype != JOLT_F32 && q_dtype != JOLT_BF16) return fail(JOLT_E_INVALID, "q_dtype");
  if (!std::isfinite(softmax_scale)) return fail(JOLT_E_INVALID, "softmax_scale not finite");
  if (check_rope(q_pos, batch, inv_freq, caches[0]->d) != JOLT_OK)
    return fail(JOLT_E_INVALID, "q_pos must lie in [0, 2^20] and inv_freq in [0, 1]");
  if (tail.cap > 0) {
    if (!tail.k || !tail.v || !tail.len) return fail(JOLT_E_INVALID, "NULL tail pointer");
    if (tail.dtype != JOLT_F32 && tail.dtype != JOLT_BF16) return fail(JOLT_E_INVALID, "tail dtype");
    for (int b = 0; b < batch; ++b)
      if (tail.len[b] < 0 || tail.len[b] > tail.cap)
        return fail(JOLT_E_INVALID, "tail_len[%d]=%d outside [0, %d]", b, tail.len[b], tail.cap);
  }
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
  const bool mfma = p.kernel == JOLT_KERNEL_MFMA;
  const bool direct = mfma && p.n_split == 1 && p.n_tsplit == 0;  // nothing to merge
  // splits per workspace row: the MFMA path keeps the tail's partials in the
  // same rows, after the split kernel's
  const int ws_splits = mfma ? p.n_split + p.n_tsplit : p.n_split;
  for (int b0 = 0; b0 < batch; b0 += kMaxBatchPerLaunch) {
    int nb = std::min(kMaxBatchPerLaunch, batch - b0);
    a.q = (const uint8_t *)q + b0 * qbytes;
    a.out = out + (size_t)b0 * c0->H_q * c0->d;
    a.ws = (float *)workspace + (size_t)b0 * c0->H_q * ws_splits * p.stride;
    a.n_tsplit = mfma ? 0 : p.n_tsplit;
    a.tail_ws = mfma || !p.n_tsplit ? nullptr
                                    : (const float *)((const uint8_t *)workspace + p.tail_off) +
                                          (size_t)b0 * c0->H_q * p.n_tsplit * (4 + c0->d);
    hipError_t e = hipSuccess;
    // the second value pass of this chunk (sequences of the classes that take it)
    V2Args v2;
    std::memset(&v2, 0, sizeof v2);
    if (p.v2) {
      v2.scores = (const float *)((const uint8_t *)workspace + p.sc_off) + (size_t)b0 * c0->H * p.sc_stride;
      v2.stats = (const float *)((const uint8_t *)workspace + p.st_off) + (size_t)b0 * c0->H * 2;
      v2.part = (float *)((uint8_t *)workspace + p.p2_off) + (size_t)b0 * p.n2split * c0->H * p.rV_max;
      v2.out = a.out;
      v2.H = c0->H;
      v2.d = c0->d;
      v2.sc_stride = p.sc_stride;
      v2.n2split = p.n2split;
      v2.split2 = p.split2;
      v2.rV_max = p.rV_max;
    }
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
      ma.ws_splits = ws_splits;
      ma.split_tokens = a.split_tokens;
      ma.stride = a.stride;
      ma.fixed_blocks = launch && launch->deterministic ? 1 : 0;
      // one split and no tail: the split kernel writes the output (and the
      // second value pass's statistics) itself, and no merge runs
      ma.out = direct ? a.out : nullptr;
      ma.stats = direct && p.v2 ? (float *)v2.stats : nullptr;
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
        int n = 0, nkt = 0, rv = 0, lds = 0, lds2 = 0;
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
          // (the logits-out variant: 8 waves, no value-rank blocks)
          lds2 = std::max(lds2, (int)mfma_lds_layout(c->d, nkt, k.bits > 0, 0, 8, true).total);
        }
        ma.nseq = n;
        ma.rV_max = rv;
        const bool two = p.v2 && v2_class(k0.bits, v0.bits, nkt, rv / 16, c0->H_q == c0->H);
        ma.scores = two ? (float *)v2.scores : nullptr;
        ma.sc_stride = two ? p.sc_stride : 0;
        if (two) {
          lds = lds2;
          for (int i = 0; i < n; ++i) {
            const jolt_cache *c = caches[b0 + ma.seq[i].slot];
            const CellDev &v = c->h_layers[layer].c[1];
            if (v.rT_pad == 0) continue;  // no value factor: nothing for the second pass
            SeqV2 &w = v2.seq[v2.nseq++];
            w.A = v.A;
            w.W2 = (const _Float16 *)v.W2;
            w.T = c->T;
            w.rT_pad = v.rT_pad;
            w.slot = ma.seq[i].slot;
          }
        }
        // XCD-aware grid (all heads of a (sequence, split) unit on one XCD)
        ma.grid8 = (a.n_split & 7) == 0 ? 1 : ((n * a.n_split) & 7) == 0 ? 2 : 0;
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
        // (with a second value pass the end event goes to its last kernel)
        if (i0 == last_class && !p.v2) ev.end = ev_last;
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
    if (p.n_tsplit > 0) {
      // the uncompressed tail: flash-decoding splits over its rows, written as
      // output-space partials [m, l, 0, 0, o/l] into the same merge
      DenseArgs da;
      std::memset(&da, 0, sizeof da);
      da.scale = softmax_scale;
      da.kv_f32 = tail.dtype == JOLT_F32;
      da.q_f32 = a.q_f32;
      da.H = c0->H;
      da.H_q = c0->H_q;
      da.Hg = a.Hg;
      da.d = c0->d;
      da.T = tail.cap;
      da.n_split = p.n_tsplit;
      da.split_tokens = p.tail_split;
      std::memcpy(da.inv_freq, a.inv_freq, sizeof da.inv_freq);
      const size_t kvb = (size_t)c0->H * tail.cap * c0->d * (da.kv_f32 ? 4 : 2);
      da.k = (const uint8_t *)tail.k + b0 * kvb;
      da.v = (const uint8_t *)tail.v + b0 * kvb;
      da.q = a.q;
      da.out = a.out;
      da.batch = nb;
      da.seq0 = b0;
      for (int i = 0; i < nb; ++i) {
        da.q_pos[i] = q_pos[b0 + i];
        da.T_seq[i] = tail.len[b0 + i];
      }
      if (mfma) {
        da.ws = a.ws;
        da.ws_splits = ws_splits;
        da.split0 = p.n_split;
      } else {
        da.ws = (float *)a.tail_ws;
        da.ws_splits = p.n_tsplit;
        da.split0 = 0;
      }
      e = jolt_launch_dense(da, nb, s);
      if (e != hipSuccess) return fail(JOLT_E_HIP, "tail kernel launch: %s", hipGetErrorString(e));
    }
    a.nseq = nb;
    if (!direct) {
      e = mfma ? jolt_launch_merge_outputs(a, nb, ws_splits, s, p.v2 ? (float *)v2.stats : nullptr)
               : jolt_launch_merge(a, nb, s);
      if (e != hipSuccess) return fail(JOLT_E_HIP, "merge kernel launch: %s", hipGetErrorString(e));
    }
    if (p.v2) {
      e = jolt_launch_value2(v2, s, ev_last);
      if (e != hipSuccess) return fail(JOLT_E_HIP, "value pass launch: %s", hipGetErrorString(e));
    }
  }
  return ok();
}

extern "C" jolt_status jolt_decode_attention(const jolt_cache *const *caches, int32_t batch,
                                             int32_t layer, const void *q, jolt_dtype q_dtype,
                                             const int32_t *q_pos, const float *inv_freq,
                                             float softmax_scale, float *out, void *workspace,
                                             size_t ws_bytes, const jolt_launch *launch,
                                             jolt_stream stream) {
  return decode_impl(caches, batch, layer, q, q_dtype, q_pos, inv_freq, softmax_scale, TailIn{},
                     out, workspace, ws_bytes, launch, stream);
}

extern "C" jolt_status jolt_decode_attention_tail(
    const jolt_cache *const *caches, int32_t batch, int32_t layer, const void *q,
    jolt_dtype q_dtype, const int32_t *q_pos, const float *inv_freq, float softmax_scale,
    const void *k_tail, const void *v_tail, jolt_dtype tail_dtype, int32_t tail_cap,
    const int32_t *tail_len, float *out, void *workspace, size_t ws_bytes,
    const jolt_launch *launch, jolt_stream stream) {
  if (tail_cap < 0 || tail_cap > kMaxPos) return fail(JOLT_E_INVALID, "tail_cap=%d", tail_cap);
  TailIn t;
  t.k = k_tail;
  t.v = v_tail;
  t.dtype = tail_dtype;
  t.cap = tail_cap;
  t.len = tail_len;
  return decode_impl(caches, batch, layer, q, q_dtype, q_pos, inv_freq, softmax_scale, t, out,
                     workspace, ws_bytes, launch, stream);
}

// ------------------------------------------------- allocation-free decode --
// The split partials of jolt_decode_attention_noalloc live in this file-scope
// device array.  Every GPU the library runs on holds its own copy (until the
// process ends); host code never passes the array's name to a kernel -- its
// per-device address comes from hipGetSymbolAddress, taken once per device
// with that device current.
static constexpr size_t kScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

static jolt_status scratch_address(void **out) {
  static std::mutex mu;
  static void *addr[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(JOLT_E_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return fail(JOLT_E_UNSUPPORTED, "device index %d >= 64", dev);
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(JOLT_E_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    addr[dev] = p;
  }
  *out = addr[dev];
  return JOLT_OK;
}

extern "C" size_t jolt_noalloc_scratch_bytes(void) { return kScratchBytes; }

extern "C" jolt_status jolt_decode_attention_noalloc(const jolt_cache *const *caches, int32_t batch,
                                                     int32_t layer, const void *q, jolt_dtype q_dtype,
                                                     const int32_t *q_pos, const float *inv_freq,
                                                     float softmax_scale, float *out,
                                                     const jolt_launch *launch, jolt_stream stream) {
  Plan p;
  // (the value factors stay in the split kernel here: the second pass needs
  // workspace for every token's logit)
  jolt_status st = plan_decode(caches, batch, layer, launch, 0, &p, false);
  if (st != JOLT_OK) return st;
  if (p.ws_bytes > kScratchBytes)
    return fail(JOLT_E_WORKSPACE,
                "this call needs %zu bytes of split partials; the allocation-free entry point "
                "holds at most %zu (use jolt_decode_attention with a workspace)",
                p.ws_bytes, kScratchBytes);
  if (batch == 0) return ok();
  void *ws = nullptr;
  st = scratch_address(&ws);
  if (st != JOLT_OK) return st;
  return decode_impl(caches, batch, layer, q, q_dtype, q_pos, inv_freq, softmax_scale, TailIn{},
                     out, ws, kScratchBytes, launch, stream, false);
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
    a.ws_splits = n_split;
    a.split0 = 0;
    for (int i = 0; i < nb; ++i) {
      a.q_pos[i] = q_pos[b0 + i];
      a.T_seq[i] = T;
    }
    hipError_t e = jolt_launch_dense(a, nb, s);
    if (e != hipSuccess) return fail(JOLT_E_HIP, "dense launch: %s", hipGetErrorString(e));
    e = jolt_launch_dense_merge(a, nb, s);
    if (e != hipSuccess) return fail(JOLT_E_HIP, "dense merge launch: %s", hipGetErrorString(e));
  }
  return ok();
}

// --------------------------------------------------------- test helpers --
extern "C" jolt_status jolt_make_rotation(uint64_t seed, int32_t d, double *out) {
  return jolt::guarded("jolt_make_rotation", [&]() -> jolt_status {
    if (!out || d < 1 || d > 4096) return fail(JOLT_E_INVALID, "out NULL or d=%d", d);
    jolt::make_rotation(seed, d, out);
    return ok();
  });
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
  if (variant < 0 || variant > 2) return fail(JOLT_E_INVALID, "variant %d not 0, 1 or 2", variant);
  const size_t nin = (size_t)n * (variant == 2 ? 2 : 1);  // input floats
  for (size_t i = 0; i < nin; ++i) {
    if (variant == 2 && (i & 1)) {
      if (!(angles[i] >= 0.0f && angles[i] <= 1.0f))
        return fail(JOLT_E_INVALID, "inv_freq %g outside [0, 1]", (double)angles[i]);
    } else if (!(std::fabs(angles[i]) < (float)kMaxPos)) {
      return fail(JOLT_E_INVALID, "angle or position %g outside (-2^20, 2^20)", (double)angles[i]);
    }
  }
  if (n == 0) return ok();
  float *d = nullptr;
  HIP_TRY(hipMalloc(&d, sizeof(float) * (nin + 2 * (size_t)n)));
  hipError_t e = hipMemcpy(d, angles, sizeof(float) * nin, hipMemcpyHostToDevice);
  if (e == hipSuccess) e = jolt_launch_sincos(d, n, d + nin, d + nin + n, variant, nullptr);
  if (e == hipSuccess) e = hipMemcpy(sin_out, d + nin, sizeof(float) * n, hipMemcpyDeviceToHost);
  if (e == hipSuccess) e = hipMemcpy(cos_out, d + nin + n, sizeof(float) * n, hipMemcpyDeviceToHost);
  hipFree(d);
  if (e != hipSuccess) return fail(JOLT_E_HIP, "debug sincos: %s", hipGetErrorString(e));
  return ok();
}
