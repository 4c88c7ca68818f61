// CPU check of the cache re-layout (layout.cpp), built with the address and
// undefined-behaviour sanitizers by tests/test_layout_cpu.py.
//
// For seeded descriptors (bf16 factors, residuals of 2, 4 and 8 bits, odd
// token counts, key and value ranks above 256, several layers per group) it
// stages the device image and reads it back the way the MFMA decode kernel
// does:
//   * key codes: the lane group's chunk of a token row, slots unpacked in
//     pairs by mantissa injection (the kernel's code_pair / unpack8 steps,
//     fp16 arithmetic included) -> must equal code - (2^b - 1)/2 of the
//     canonical LSB-first packing, for every (layer, head, token, feature);
//   * value codes: the lane records of a 16-token block, pairs per feature
//     block -> the same;
//   * every bit of a code section that no read touches must be zero;
//   * A_K fragments and A_V tiles at the kernel's addresses -> fp16(A * a_s);
//   * W2[h] = B G[h]^T / a_s within fp16 rounding, padding columns zero.
// Prints "layout check OK" and exits 0, or reports the first mismatch.
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "layout.h"

using namespace jolt;

static uint64_t g_state = 0x9E3779B97F4A7C15ULL;
static uint32_t rnd() {
  g_state = g_state * 6364136223846793005ULL + 1442695040888963407ULL;
  return (uint32_t)(g_state >> 33);
}
static float rndf() { return ((float)rnd() / 2147483648.0f) - 1.0f; }
static uint16_t to_bf16(float x) {
  uint32_t u;
  std::memcpy(&u, &x, 4);
  u += 0x7FFF + ((u >> 16) & 1);
  return (uint16_t)(u >> 16);
}
static float bf16f(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

static int fails = 0;
#define CHECK(cond, ...)                         \
  do {                                           \
    if (!(cond)) {                               \
      if (fails++ < 10) {                        \
        std::fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
        std::fprintf(stderr, __VA_ARGS__);       \
        std::fprintf(stderr, "\n");              \
      }                                          \
    }                                            \
  } while (0)

// The kernel's pair decode: codes at bit offsets sh and sh + 16 of w become
// the fp16 pair (c - L/2): mantissa 2c + 1 injected under 0x6001 (512.5),
// then 512 + 2^(b-1) subtracted.
static void code_pair(uint32_t w, int sh, int b, float out[2]) {
  const uint32_t m = (((1u << b) - 1u) << 1) * 0x10001u;
  uint32_t x = sh == 0 ? (w << 1) : (w >> (sh - 1));
  x = (x & m) | 0x60016001u;
  const _Float16 bias = (_Float16)(-(512.0f + (float)(1 << (b - 1))));
  uint16_t lo = (uint16_t)(x & 0xFFFF), hi = (uint16_t)(x >> 16);
  _Float16 a, c;
  std::memcpy(&a, &lo, 2);
  std::memcpy(&c, &hi, 2);
  out[0] = (float)(_Float16)(a + bias);
  out[1] = (float)(_Float16)(c + bias);
}

struct HostCell {
  int rT, rF, bits;
  std::vector<uint16_t> A, B, G;
  std::vector<uint8_t> codes;
  std::vector<float> scales;
};

static int canon(const uint8_t *row, int i, int b) {
  const int per = 8 / b;
  return (row[i / per] >> ((i % per) * b)) & ((1 << b) - 1);
}

// One case: groups of sizes gsz, allocation per group (K, V).
static void run_case(int T, int H, int d, const std::vector<int> &gsz,
                     const std::vector<int> &alloc /* 6 per group: rT rF b for K, V */) {
  const int ng = (int)gsz.size();
  std::vector<int32_t> starts(ng + 1, 0);
  for (int g = 0; g < ng; ++g) starts[g + 1] = starts[g] + gsz[g];
  std::vector<HostCell> hc(2 * ng);
  std::vector<jolt_cell> cells(2 * ng);
  for (int g = 0; g < ng; ++g)
    for (int tau = 0; tau < 2; ++tau) {
      HostCell &c = hc[2 * g + tau];
      c.rT = alloc[6 * g + 3 * tau];
      c.rF = alloc[6 * g + 3 * tau + 1];
      c.bits = alloc[6 * g + 3 * tau + 2];
      c.A.resize((size_t)T * c.rT);
      for (auto &x : c.A) x = to_bf16(rndf() * 0.05f);
      c.B.resize((size_t)d * c.rF);
      for (auto &x : c.B) x = to_bf16(rndf() * 0.3f);
      c.G.resize((size_t)gsz[g] * H * c.rT * c.rF);
      for (auto &x : c.G) x = to_bf16(rndf() * 4.0f);
      if (c.bits) {
        c.codes.resize((size_t)gsz[g] * H * T * d * c.bits / 8);
        for (auto &x : c.codes) x = (uint8_t)rnd();
        c.scales.resize((size_t)gsz[g] * H * T);
        for (auto &x : c.scales) x = 1e-3f * (1.0f + rndf() * 0.5f);
      }
      jolt_cell &jc = cells[2 * g + tau];
      jc.r_T = c.rT;
      jc.r_F = c.rF;
      jc.bits = c.bits;
      jc.A = c.A.data();
      jc.B = c.B.data();
      jc.G = c.G.data();
      jc.codes = c.bits ? c.codes.data() : nullptr;
      jc.scales = c.bits ? c.scales.data() : nullptr;
    }
  jolt_cache_desc desc;
  desc.n_layers = starts[ng];
  desc.n_groups = ng;
  desc.n_kv_heads = H;
  desc.n_q_heads = H;
  desc.head_dim = d;
  desc.T = T;
  desc.group_start = starts.data();
  desc.factor_dtype = JOLT_BF16;
  desc.rotation_seed = 7;
  desc.cells = cells.data();

  Staged S;
  stage_cache(&desc, &S, 3);
  const int T_pad = S.T_pad;
  CHECK(T_pad % kTokPad == 0 && T_pad >= T && T_pad < T + kTokPad, "T_pad %d", T_pad);
  const uint8_t *buf = S.buf.data();

  for (int g = 0; g < ng; ++g)
    for (int tau = 0; tau < 2; ++tau) {
      const HostCell &c = hc[2 * g + tau];
      const CellMeta &m = S.cells[2 * g + tau];
      const CellOffsets &o = S.offs[2 * g + tau];
      CHECK(m.rT_pad == pad_rank(c.rT) && m.rT_pad % 32 == 0 && m.rT_pad >= c.rT, "rT_pad");
      // A at the kernel's addresses.  Keys as the MFMA kernel's fetch forms
      // them: lane (lr, lg) of the 16 tokens from tb reads, for 32-rank step
      // ks, the 16 bytes at tb 64 KT + 1024 ks + 16 (4 lr + lg), element j
      // being rank 32 ks + 8 lg + j of token tb + lr (KT = rT_pad / 32).
      auto ak_fetch = [&](int t, int r) -> size_t {
        const int KT = m.rT_pad / 32, tb = t & ~15, lr = t & 15, ks = r / 32, lg = (r / 8) & 3,
                  j = r & 7;
        return (size_t)tb * 64 * KT + 1024 * (size_t)ks + 16 * (size_t)(4 * lr + lg) + 2 * (size_t)j;
      };
      for (int t = 0; t < T; ++t)
        for (int r = 0; r < m.rT_pad; ++r) {
          const size_t at = tau == 0 ? o.A + ak_fetch(t, r) : o.A + 2 * av_index(t, r, m.rT_pad);
          _Float16 v;
          std::memcpy(&v, buf + at, 2);
          const float want = r < c.rT ? (float)(_Float16)(bf16f(c.A[(size_t)t * c.rT + r]) * (float)m.a_s) : 0.0f;
          CHECK((float)v == want, "A g%d tau%d t%d r%d: %g vs %g", g, tau, t, r, (double)(float)v, (double)want);
        }
      for (int lp = 0; lp < gsz[g]; ++lp) {
        // W2
        if (c.rT > 0) {
          const int w2_row = m.rT_pad + (tau == 0 ? kRowPad : 0);
          for (int h = 0; h < H; ++h)
            for (int f = 0; f < d; ++f)
              for (int r = 0; r < w2_row; ++r) {
                _Float16 v;
                std::memcpy(&v, buf + o.W2[lp] + 2 * (((size_t)h * d + f) * w2_row + r), 2);
                double want = 0.0;
                if (r < c.rT)
                  for (int j = 0; j < c.rF; ++j)
                    want += (double)bf16f(c.B[(size_t)f * c.rF + j]) *
                            bf16f(c.G[(((size_t)lp * H + h) * c.rT + r) * c.rF + j]);
                want /= m.a_s;
                CHECK(std::fabs((double)(float)v - want) <= 1e-3 * std::fabs(want) + 1e-7,
                      "W2 g%d tau%d lp%d h%d f%d r%d: %g vs %g", g, tau, lp, h, f, r,
                      (double)(float)v, want);
              }
        }
        if (!c.bits) continue;
        const int b = c.bits, rowb = d * b / 8, L2 = 1 << (b - 1);
        const uint8_t *C = buf + o.codes[lp];
        const size_t csize = (size_t)H * T_pad * rowb;
        std::vector<uint8_t> seen(csize * 8, 0);  // bits a read touches
        auto mark = [&](size_t byte, int sh) {
          for (int k = 0; k < b; ++k) seen[(byte + (sh + k) / 8) * 8 + (sh + k) % 8] = 1;
        };
        for (int h = 0; h < H; ++h)
          for (int t = 0; t < T; ++t) {
            const uint8_t *row = c.codes.data() + (((size_t)lp * H + h) * T + t) * rowb;
            float sc;
            std::memcpy(&sc, buf + o.scales[lp] + 4 * ((size_t)h * T_pad + t), 4);
            CHECK(sc == c.scales[((size_t)lp * H + h) * T + t], "scale");
            if (tau == 0) {
              // lane group lg's chunk of the row, read as the kernel reads
              // it: chunks of 8 bytes in place in the row, wider ones as
              // 16-byte pieces, piece x of lane (t & 15, lg) at 1024 x +
              // 16 (4 (t & 15) + lg) from the 16-token block's first row;
              // residual step j unpacks slots 8 j .. 8 j + 7 = features
              // 32 j + 8 lg + e
              const int cb = d * b / 32, npair = 16 / b;
              for (int lg = 0; lg < 4; ++lg) {
                auto word_at = [&](int dw) -> size_t {
                  if (cb <= 8) return ((size_t)h * T_pad + t) * rowb + (size_t)lg * cb + 4 * dw;
                  const size_t blk = ((size_t)h * T_pad + (t & ~15)) * rowb;
                  return blk + 1024 * (size_t)(dw / 4) + 16 * (size_t)(4 * (t & 15) + lg) + 4 * (dw % 4);
                };
                for (int j = 0; j < d / 32; ++j)
                  for (int p = 0; p < 4; ++p) {
                    const int P = 4 * j + p;
                    uint32_t w;
                    std::memcpy(&w, C + word_at(P / npair), 4);
                    float v[2];
                    code_pair(w, b * (P % npair), b, v);
                    for (int e = 0; e < 2; ++e) {
                      const int i = 32 * j + 8 * lg + 2 * p + e;
                      mark(word_at(P / npair), b * (P % npair) + 16 * e);
                      CHECK(v[e] == (float)canon(row, i, b) - L2 + 0.5f,
                            "K code lp%d h%d t%d i%d b%d: %g vs %d", lp, h, t, i, b, (double)v[e], canon(row, i, b));
                    }
                  }
              }
            }
          }
        if (tau == 1) {
          // lane (lr, lg) of a 16-token block: record (lr*4 + lg); feature
          // block fb gives pairs (tokens 4 lg, 4 lg + 1) and (4 lg + 2, 4 lg + 3)
          // of feature 16 fb + lr
          const int vrec = d * b / 32, npair = 16 / b;
          for (int h = 0; h < H; ++h)
            for (int tb = 0; tb < T_pad / 16; ++tb)
              for (int lr = 0; lr < 16; ++lr)
                for (int lg = 0; lg < 4; ++lg) {
                  const size_t e0 = (((size_t)h * (T_pad >> 4) + tb) * 64 + lr * 4 + lg) * vrec;
                  for (int fb = 0; fb < d / 16; ++fb)
                    for (int half = 0; half < 2; ++half) {
                      const int P = 2 * fb + half;
                      uint32_t w;
                      std::memcpy(&w, C + e0 + 4 * (P / npair), 4);
                      float v[2];
                      code_pair(w, b * (P % npair), b, v);
                      for (int e = 0; e < 2; ++e) {
                        const int t = 16 * tb + 4 * lg + 2 * half + e, f = 16 * fb + lr;
                        if (t >= T) {
                          CHECK(v[e] == -L2 + 0.5f, "V pad code nonzero h%d t%d f%d", h, t, f);
                          continue;
                        }
                        mark(e0 + 4 * (P / npair), b * (P % npair) + 16 * e);
                        const uint8_t *row = c.codes.data() + (((size_t)lp * H + h) * T + t) * rowb;
                        CHECK(v[e] == (float)canon(row, f, b) - L2 + 0.5f,
                              "V code lp%d h%d t%d f%d b%d: %g vs %d", lp, h, t, f, b, (double)v[e], canon(row, f, b));
                      }
                    }
                }
        }
        // no stray bits anywhere in the section
        for (size_t x = 0; x < csize * 8; ++x)
          if (!seen[x]) CHECK(((C[x / 8] >> (x % 8)) & 1) == 0, "stray bit at byte %zu (g%d tau%d lp%d)", x / 8, g, tau, lp);
      }
    }
  std::printf("case T=%d H=%d groups=%d: %d failures so far\n", T, H, ng, fails);
}

// The MFMA decode kernel's LDS layout (mfma_lds_layout, shared by the host's
// launch size and the kernel): for every launch class, the arrays live during
// the token-block loop are pairwise disjoint, so are those live after it, and
// all end within the size the host requests.
static void check_mfma_lds() {
  struct R { uint32_t b, e; };
  auto disjoint = [](R x, R y) { return x.e <= y.b || y.e <= x.b || x.b == x.e || y.b == y.e; };
  const int kts[] = {0, 1, 2, 3, 4, 5, 6, 7, 8, 10, 12, 14, 16};
  int n = 0;
  for (int kt : kts)
    for (int pi = 0; pi < 2; ++pi)
      for (int nmv = 0; nmv <= 32; ++nmv)
        for (int waves = 4; waves <= 8; waves += 4)
          for (int hg1 = 0; hg1 < 2; ++hg1) {
            const jolt::MfmaLds L = jolt::mfma_lds_layout(128, kt, pi, nmv, waves, hg1);
            const R kp{0, L.kpath}, red{L.red, L.red + 128u * waves}, ifr{L.ifr, L.ifr + 512},
                qf{L.qf, L.qf + 6144}, ql{L.ql, hg1 ? L.ql : L.ql + 6144}, ctr{L.ctr, L.ctr + 4},
                park{0, L.park}, xa{L.xa, L.xa + L.xa_bytes};
            const R loop[] = {kp, red, ifr, qf, ql, ctr};
            const R after[] = {park, xa, red, ifr, qf, ctr};
            for (int i = 0; i < 6; ++i)
              for (int j = i + 1; j < 6; ++j) {
                CHECK(disjoint(loop[i], loop[j]), "LDS loop regions %d/%d overlap (kt%d pi%d nmv%d w%d hg1 %d)",
                      i, j, kt, pi, nmv, waves, hg1);
                CHECK(disjoint(after[i], after[j]), "LDS post-loop regions %d/%d overlap (kt%d pi%d nmv%d w%d hg1 %d)",
                      i, j, kt, pi, nmv, waves, hg1);
              }
            for (const R &r : loop) CHECK(r.e <= L.total, "LDS region past the launch size (kt%d nmv%d)", kt, nmv);
            for (const R &r : after) CHECK(r.e <= L.total, "LDS region past the launch size (kt%d nmv%d)", kt, nmv);
            CHECK(L.total % 4 == 0 && L.ctr % 4 == 0 && L.xa % 16 == 0 && L.qf % 16 == 0, "LDS alignment");
            // a sequence launched with fewer waves or as the one-query variant
            // needs no more LDS than the host's per-sequence size
            CHECK(jolt::mfma_lds_layout(128, kt, pi, nmv, 4, hg1).total <= jolt::mfma_lds_layout(128, kt, pi, nmv, waves, hg1).total &&
                      jolt::mfma_lds_layout(128, kt, pi, nmv, waves, true).total <= jolt::mfma_lds_layout(128, kt, pi, nmv, waves, hg1).total,
                  "LDS size not monotone (kt%d nmv%d)", kt, nmv);
            ++n;
          }
  std::printf("mfma LDS layouts: %d classes checked, %d failures so far\n", n, fails);
}

int main() {
  const int d = 128;
  // (T, H, group sizes, allocation)
  run_case(37, 3, d, {2}, {16, 16, 2, 32, 16, 4});
  run_case(301, 2, d, {1, 2}, {200, 64, 8, 96, 32, 2, 288, 48, 4, 300, 96, 8});
  run_case(1, 3, d, {1}, {1, 16, 4, 1, 16, 8});
  run_case(1111, 2, d, {3}, {512, 96, 4, 300, 64, 2});
  run_case(130, 2, d, {1}, {0, 0, 8, 0, 0, 4});
  check_mfma_lds();
  if (fails) {
    std::printf("layout check FAILED (%d)\n", fails);
    return 1;
  }
  std::printf("layout check OK\n");
  return 0;
}
