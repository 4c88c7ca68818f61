// Generic split-T decode kernel, split merge/finalize, dense decode kernel and
// the debug unpack kernel of libjolt (gfx950).
//
// What is computed: decode attention over a JoLT-compressed cache ("A JoLT
// for the KV cache", arXiv 2607.12550v4 summary, Abstract and §4.5: attention
// directly over the stored factors and packed residuals, keys rebuilt per
// tile because RoPE does not commute with the factorisation).  The value path
// uses linearity: each split keeps a = sum_t p_t A_V[t] and c = sum_t p_t
// deq_V[t]; the merge forms o = (a G_V) B_V^T + c Pi^T.
//
// The generic kernel is plain SIMT (fp32 arithmetic, LDS tiles of 32
// tokens).  It serves float32 caches and shapes the MFMA kernel does not take.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include "jolt_internal.h"
#include "trig.h"

using namespace jolt;

namespace {

constexpr int kTT = 32;  // tokens per generic tile
constexpr int kGenStage = kMaxD * (kMaxD + 2);  // floats of LDS for the generic kernel's key-side matrices
constexpr int kMergeChunk = 2048;

__device__ inline float bf16f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

template <bool F32>
__device__ inline float ldf(const void *p, size_t i) {
  if constexpr (F32)
    return ((const float *)p)[i];
  else
    return bf16f(((const uint16_t *)p)[i]);
}

// A element (keys or values): float32 caches as stored; bf16 caches keep A as fp16(A * s).
template <bool F32>
__device__ inline float ldAk(const CellDev &K, size_t i) {
  if constexpr (F32)
    return ((const float *)K.A)[i];
  else
    return (float)((const _Float16 *)K.A)[i] * K.a_inv;
}

__device__ inline float ldq(const void *q, size_t i, bool f32) {
  return f32 ? ((const float *)q)[i] : bf16f(((const uint16_t *)q)[i]);
}

__device__ inline int k_code(const CellDev &c, int h, int t, int i, int T_pad, int d) {
  size_t at;
  int sh;
  kcode_pos(h, t, i, c.bits, T_pad, d, &at, &sh);
  const uint32_t w = *(const uint32_t *)(c.codes + at);
  return (w >> sh) & ((1u << c.bits) - 1u);
}

__device__ inline int v_code(const CellDev &c, int h, int t, int i, int T_pad, int d) {
  const int b = c.bits;
  size_t at;
  int sh;
  vcode_pos(h, t, i, b, T_pad, d, &at, &sh);
  uint32_t w = *(const uint32_t *)(c.codes + at);
  return (w >> sh) & ((1u << b) - 1u);
}

__device__ inline float deq(int code, int bits, float scale) {
  return ((float)code - 0.5f * (float)((1 << bits) - 1)) * scale;
}

// RoPE angle of pair i at position t: the float32 product fl32(t * inv_freq[i]).
__device__ inline void rope_cs(int t, float f, float *c, float *s) { rope_angle_cs(t, f, c, s); }

// ------------------------------------------------------------ generic --
template <bool F32>
__global__ __launch_bounds__(256) void decode_generic(DecodeArgs a) {
  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const SeqArg sa = a.seq[b];
  const LayerDev &L = *sa.layer;
  const CellDev &K = L.c[0], &V = L.c[1];
  const int T = sa.T, T_pad = L.T_pad, d = a.d, Hg = a.Hg, half = d / 2;
  const int t0 = split * a.split_tokens, t1 = min(T, t0 + a.split_tokens);

  __shared__ float qr[kMaxHg][kMaxD];
  __shared__ float P[kTT][kMaxD];
  __shared__ float X[kTT][kMaxD];
  __shared__ float Kt[kTT][kMaxD];
  __shared__ float S[kMaxHg][kTT];
  __shared__ float cacc[kMaxHg][kMaxD];
  __shared__ float m_s[kMaxHg], l_s[kMaxHg], al_s[kMaxHg];
  // The key-side matrices every tile reads, staged once per workgroup as
  // float: Pi (b_K > 0), then B_K and G_K[h] where they still fit (read from
  // memory otherwise).  Each key element reads a whole row of them, so from
  // memory the tile loop waits on one load per multiply-add.  Rows carry one
  // float of padding: the threads of a wave read different rows at the same
  // column, which would otherwise all fall on one LDS bank.
  __shared__ float stage[kGenStage];

  float *part0 = a.ws + ((size_t)(b * a.H_q + h * Hg) * a.n_split + split) * a.stride;
  const size_t ustride = (size_t)a.n_split * a.stride;

  if (t0 >= t1) {  // empty split (shorter sequence in the batch)
    for (int u = tid; u < Hg; u += 256) {
      part0[u * ustride + 0] = -INFINITY;
      part0[u * ustride + 1] = 0.0f;
    }
    return;
  }

  // query heads of this KV head, rotated to q_pos
  for (int x = tid; x < Hg * half; x += 256) {
    int u = x / half, i = x % half;
    size_t qi = ((size_t)b * a.H_q + h * Hg + u) * d;
    float lo = ldq(a.q, qi + i, a.q_f32), hi = ldq(a.q, qi + i + half, a.q_f32);
    float c, s;
    rope_cs(sa.q_pos, a.inv_freq[i], &c, &s);
    qr[u][i] = lo * c - hi * s;
    qr[u][i + half] = hi * c + lo * s;
  }
  for (int x = tid; x < Hg * d; x += 256) cacc[x / d][x % d] = 0.0f;
  for (int u = tid; u < Hg; u += 256) {
    m_s[u] = -INFINITY;
    l_s[u] = 0.0f;
  }
  for (int x = tid; x < Hg * V.rT_pad; x += 256)
    part0[(x / V.rT_pad) * ustride + 4 + (x % V.rT_pad)] = 0.0f;
  const int sPi = d + 1, sB = K.rF + 1, sG = K.rT + 1;  // staged row strides
  const int nPi = K.bits ? d * sPi : 0, nB = d * sB, nG = K.rF * sG;
  const bool bL = nPi + nB <= kGenStage, gL = bL && nPi + nB + nG <= kGenStage;
  float *const Pis = stage, *const Bs = stage + nPi, *const Gs = stage + nPi + nB;
  if (K.bits)
    for (int x = tid; x < d * d; x += 256) Pis[(x / d) * sPi + x % d] = L.Pi[x];
  if (bL)
    for (int x = tid; x < d * K.rF; x += 256)
      Bs[(x / K.rF) * sB + x % K.rF] = ldf<F32>(K.B, (size_t)(x / K.rF) * K.rF_pad + x % K.rF);
  if (gL)
    for (int x = tid; x < K.rF * K.rT; x += 256)
      Gs[(x / K.rT) * sG + x % K.rT] = ldf<F32>(K.G, ((size_t)h * K.rF_pad + x / K.rT) * K.rT_pad + x % K.rT);
  __syncthreads();

  const float Lk = 0.5f * (float)((1 << K.bits) - 1);
  for (int tt = t0; tt < t1; tt += kTT) {
    const int nt = min(kTT, t1 - tt);
    // the tile's A_K rows, staged in Kt (written only after P) when they fit
    const bool aL = gL && K.rT <= kMaxD;
    if (aL) {
      for (int x = tid; x < nt * K.rT; x += 256)
        Kt[x / K.rT][x % K.rT] = ldAk<F32>(K, ak_index(tt + x / K.rT, x % K.rT, K.rT_pad));
      __syncthreads();
    }
    // P = A_K[t] G_K  (t < nt, j < r_F)
    for (int x = tid; x < nt * K.rF; x += 256) {
      int t = x / K.rF, j = x % K.rF;
      float acc = 0.0f;
      if (aL)
        for (int r = 0; r < K.rT; ++r) acc += Kt[t][r] * Gs[j * sG + r];
      else if (gL)
        for (int r = 0; r < K.rT; ++r) acc += ldAk<F32>(K, ak_index(tt + t, r, K.rT_pad)) * Gs[j * sG + r];
      else
        for (int r = 0; r < K.rT; ++r)
          acc += ldAk<F32>(K, ak_index(tt + t, r, K.rT_pad)) *
                 ldf<F32>(K.G, ((size_t)h * K.rF_pad + j) * K.rT_pad + r);
      P[t][j] = acc;
    }
    // key residual in the rotated basis
    if (K.bits)
      for (int x = tid; x < nt * d; x += 256) {
        int t = x / d, i = x % d;
        X[t][i] = ((float)k_code(K, h, tt + t, i, T_pad, d) - Lk) *
                  K.scales[(size_t)h * T_pad + tt + t];
      }
    __syncthreads();
    // K_pre = P B_K^T + deq Pi^T
    for (int x = tid; x < nt * d; x += 256) {
      int t = x / d, f = x % d;
      float acc = 0.0f;
      if (bL)
        for (int j = 0; j < K.rF; ++j) acc += P[t][j] * Bs[f * sB + j];
      else
        for (int j = 0; j < K.rF; ++j) acc += P[t][j] * ldf<F32>(K.B, (size_t)f * K.rF_pad + j);
      if (K.bits)
        for (int i = 0; i < d; ++i) acc += X[t][i] * Pis[f * sPi + i];
      Kt[t][f] = acc;
    }
    __syncthreads();
    // RoPE at each token's own position
    for (int x = tid; x < nt * half; x += 256) {
      int t = x / half, i = x % half;
      float c, s;
      rope_cs(tt + t, a.inv_freq[i], &c, &s);
      float lo = Kt[t][i], hi = Kt[t][i + half];
      Kt[t][i] = lo * c - hi * s;
      Kt[t][i + half] = hi * c + lo * s;
    }
    __syncthreads();
    for (int x = tid; x < Hg * nt; x += 256) {
      int u = x / nt, t = x % nt;
      float acc = 0.0f;
      for (int f = 0; f < d; ++f) acc += qr[u][f] * Kt[t][f];
      S[u][t] = a.scale * acc;
    }
    // value residual (rotated basis) into X
    const float Lv = 0.5f * (float)((1 << V.bits) - 1);
    __syncthreads();
    if (V.bits)
      for (int x = tid; x < nt * d; x += 256) {
        int t = x / d, i = x % d;
        X[t][i] = ((float)v_code(V, h, tt + t, i, T_pad, d) - Lv) *
                  V.scales[(size_t)h * T_pad + tt + t];
      }
    // the tile's A_V rows, staged in P (no longer read) when they fit
    const bool avL = V.rT <= kMaxD;
    if (avL)
      for (int x = tid; x < nt * V.rT; x += 256)
        P[x / V.rT][x % V.rT] = ldAk<F32>(V, av_index(tt + x / V.rT, x % V.rT, V.rT_pad));
    // online softmax
    if (tid < Hg) {
      int u = tid;
      float mt = -INFINITY;
      for (int t = 0; t < nt; ++t) mt = fmaxf(mt, S[u][t]);
      float mn = fmaxf(m_s[u], mt);
      float al = expf(m_s[u] - mn);
      float sum = 0.0f;
      for (int t = 0; t < nt; ++t) {
        float p = expf(S[u][t] - mn);
        S[u][t] = p;
        sum += p;
      }
      l_s[u] = al * l_s[u] + sum;
      m_s[u] = mn;
      al_s[u] = al;
    }
    __syncthreads();
    if (V.bits)
      for (int x = tid; x < Hg * d; x += 256) {
        int u = x / d, i = x % d;
        float acc = 0.0f;
        for (int t = 0; t < nt; ++t) acc += S[u][t] * X[t][i];
        cacc[u][i] = al_s[u] * cacc[u][i] + acc;
      }
    for (int x = tid; x < Hg * V.rT; x += 256) {
      int u = x / V.rT, r = x % V.rT;
      float acc = 0.0f;
      if (avL)
        for (int t = 0; t < nt; ++t) acc += S[u][t] * P[t][r];
      else
        for (int t = 0; t < nt; ++t) acc += S[u][t] * ldAk<F32>(V, av_index(tt + t, r, V.rT_pad));
      float *pa = part0 + u * ustride + 4 + r;
      *pa = al_s[u] * *pa + acc;
    }
    __syncthreads();
  }
  for (int x = tid; x < Hg * d; x += 256) {
    int u = x / d, i = x % d;
    part0[u * ustride + 4 + a.rV_max + i] = cacc[u][i];
  }
  for (int u = tid; u < Hg; u += 256) {
    part0[u * ustride + 0] = m_s[u];
    part0[u * ustride + 1] = l_s[u];
  }
}

// -------------------------------------------------------------- merge --
// One workgroup per (sequence, query head j): combine the split partials
// (weights w_s = exp(m_s - max m), a = sum w_s a_s / sum w_s l_s, c alike),
// then finalize o = (a G_V[h]) B_V^T + c Pi^T with h = j / Hg.
__device__ inline float block_reduce(float v, float *red, bool is_max) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    float w = __shfl_xor(v, o);
    v = is_max ? fmaxf(v, w) : v + w;
  }
  if ((tid & 63) == 0) red[tid >> 6] = v;
  __syncthreads();
  float r = red[0];
  for (int i = 1; i < (int)(blockDim.x >> 6); ++i) r = is_max ? fmaxf(r, red[i]) : r + red[i];
  __syncthreads();
  return r;
}

// Weighted sum over splits of partial column `off` for columns
// col0 + tid, col0 + tid + nthreads, ...: loads are issued in batches of 16
// splits so that many are in flight per thread.
__device__ inline void split_columns(const float *pb, int st, int ns, const float *w_s,
                                     int ncol, int off0, float inv, float *dst, int tid,
                                     int nthreads) {
  for (int x = tid; x < ncol; x += nthreads) {
    float acc = 0.0f;
    for (int s0 = 0; s0 < ns; s0 += 16) {
      float v[16];
#pragma unroll
      for (int k = 0; k < 16; ++k) v[k] = s0 + k < ns ? pb[(size_t)(s0 + k) * st + off0 + x] : 0.0f;
#pragma unroll
      for (int k = 0; k < 16; ++k)
        if (s0 + k < ns && w_s[s0 + k] > 0.0f) acc += w_s[s0 + k] * v[k];
    }
    dst[x] = acc * inv;
  }
}

template <bool F32>
__global__ __launch_bounds__(256) void merge_finalize(DecodeArgs a) {
  const int j = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int Hg = a.Hg, h = j / Hg, d = a.d, ns = a.n_split;
  const SeqArg sa = a.seq[b];
  const LayerDev &L = *sa.layer;
  const CellDev &V = L.c[1];
  __shared__ float w_s[kMaxSplits];
  __shared__ float av[kMergeChunk];
  __shared__ float cv[kMaxD];
  __shared__ float yv[2][kMaxD];
  __shared__ float ov[2][kMaxD];
  __shared__ float red[8];
  __shared__ __attribute__((aligned(16))) float mat[kMaxD * kMaxD];  // staged Pi^T or B_V^T
  const float *pb = a.ws + ((size_t)(b * a.H_q + j) * ns) * a.stride;
  const int st = a.stride;

  // uncompressed-tail partials [m, l, 0, 0, o/l] of this (sequence, query
  // head), if any: they join the same softmax
  const int nts = a.n_tsplit, tst = 4 + d;
  const float *tp = nts > 0 ? a.tail_ws + (size_t)(b * a.H_q + j) * nts * tst : nullptr;
  __shared__ float wt_s[kMaxTailSplits];
  float mx = -INFINITY;
  for (int s = tid; s < ns; s += 256) {
    float m = pb[(size_t)s * st];
    w_s[s] = m;
    mx = fmaxf(mx, m);
  }
  for (int s = tid; s < nts; s += 256) mx = fmaxf(mx, tp[(size_t)s * tst]);
  mx = block_reduce(mx, red, true);
  float ls = 0.0f;
  for (int s = tid; s < ns; s += 256) {
    float m = w_s[s];
    float w = (m == -INFINITY) ? 0.0f : __expf(m - mx);
    w_s[s] = w;
    ls += w * pb[(size_t)s * st + 1];
  }
  for (int s = tid; s < nts; s += 256) {
    const float m = tp[(size_t)s * tst];
    const float w = (m == -INFINITY) ? 0.0f : __expf(m - mx) * tp[(size_t)s * tst + 1];
    wt_s[s] = w;  // weight of the split's normalised output o/l
    ls += w;
  }
  ls = block_reduce(ls, red, false);  // also orders the w_s / wt_s writes
  const float inv = 1.0f / ls;

  split_columns(pb, st, ns, w_s, d, 4 + a.rV_max, inv, cv, tid, 256);
  // y = a G_V[h]: two thread halves split the rank sum, chunk by chunk
  const int na = V.rT, half = tid >> 7, jj = tid & 127;
  float yacc = 0.0f;
  for (int r0 = 0; r0 < na; r0 += kMergeChunk) {
    const int nr = min(kMergeChunk, na - r0);
    __syncthreads();
    split_columns(pb, st, ns, w_s, nr, 4 + r0, inv, av, tid, 256);
    __syncthreads();
    if (jj < V.rF) {
      float g[8];
      for (int r = half; r < nr; r += 16) {
#pragma unroll
        for (int k = 0; k < 8; ++k)
          g[k] = r + 2 * k < nr ? ldf<F32>(V.G, ((size_t)h * V.rT_pad + r0 + r + 2 * k) * V.rF_pad + jj)
                                : 0.0f;
#pragma unroll
        for (int k = 0; k < 8; ++k)
          if (r + 2 * k < nr) yacc += av[r + 2 * k] * g[k];
      }
    }
  }
  yv[half][jj] = yacc;
  __syncthreads();
  if (tid < 128) yv[0][tid] += yv[1][tid];
  // o = y B_V^T + c Pi^T with each matrix staged in LDS by bulk loads
  float acc = 0.0f;
  const int f = tid & 127, part = tid >> 7;
  if (V.rF > 0) {
    __syncthreads();
    stage_rows((uint8_t *)mat, 4 * d, (const uint8_t *)V.Bt, V.rF, d / 4, tid, 256);
    __syncthreads();
    if (f < d)
      for (int q = part; q < V.rF; q += 2) acc += yv[0][q] * mat[q * d + f];
  }
  if (V.bits) {
    __syncthreads();
    stage_rows((uint8_t *)mat, 4 * d, (const uint8_t *)L.PiT, d, d / 4, tid, 256);
    __syncthreads();
    if (f < d)
      for (int i = part; i < d; i += 2) acc += cv[i] * mat[i * d + f];
  }
  // the tail's share: sum over its splits of w o (o already divided by l)
  if (f < d)
    for (int s = part; s < nts; s += 2)
      if (wt_s[s] > 0.0f) acc += wt_s[s] * inv * tp[(size_t)s * tst + 4 + f];
  if (f < d) ov[part][f] = acc;
  __syncthreads();
  if (tid < d) a.out[((size_t)b * a.H_q + j) * d + tid] = ov[0][tid] + ov[1][tid];
}

// -------------------------------------------------------------- dense --
// Flash-decoding over post-RoPE bf16/fp32 K and V.  A group of D/8 lanes owns
// one token at a time (8 features per lane, one 16-byte load); each group
// walks U consecutive tokens per step and keeps its own online-softmax state,
// merged across groups at the end of the split.
template <int D, int HG, bool KV32>
__global__ __launch_bounds__(256) void dense_split(DenseArgs a) {
  constexpr int LPT = D / 8, TPP = 256 / LPT, U = 4;
  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int tg = tid / LPT, li = tid % LPT;
  const int Hg = a.Hg, T = a.T;
  const int t0 = split * a.split_tokens, t1 = min(a.T_seq[b], t0 + a.split_tokens);
  const int qpos = a.q_pos[b];
  // the workgroup's query heads rotated to q_pos (one pair per thread), scaled
  __shared__ float qs[HG][D];
  for (int x = tid; x < Hg * (D / 2); x += 256) {
    const int u = x / (D / 2), i = x % (D / 2);
    const size_t qi = ((size_t)b * a.H_q + h * Hg + u) * D;
    float c, s;
    rope_cs(qpos, a.inv_freq[i], &c, &s);
    const float lo = ldq(a.q, qi + i, a.q_f32), hi = ldq(a.q, qi + i + D / 2, a.q_f32);
    qs[u][i] = (lo * c - hi * s) * a.scale;
    qs[u][i + D / 2] = (hi * c + lo * s) * a.scale;
  }
  __syncthreads();
  float qv[HG][8];
#pragma unroll
  for (int u = 0; u < HG; ++u)
#pragma unroll
    for (int e = 0; e < 8; ++e) qv[u][e] = u < Hg ? qs[u][8 * li + e] : 0.0f;
  float m[HG], l[HG], acc[HG][8];
#pragma unroll
  for (int u = 0; u < HG; ++u) {
    m[u] = -INFINITY;
    l[u] = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[u][e] = 0.0f;
  }
  const size_t base = ((size_t)b * a.H + h) * T * D;
  for (int tb = t0 + tg * U; tb < t1; tb += TPP * U) {
    float kf[U][8], vf[U][8];
#pragma unroll
    for (int k = 0; k < U; ++k) {
      int t = tb + k;
      if (t < t1) {
        size_t off = base + (size_t)t * D + 8 * li;
        if constexpr (KV32) {
          gptr<gf32x4> kp = gp<gf32x4>(a.k), vp = gp<gf32x4>(a.v);
          gf32x4 k0 = kp[off / 4], k1 = kp[off / 4 + 1], v0 = vp[off / 4], v1 = vp[off / 4 + 1];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            kf[k][e] = k0[e];
            kf[k][e + 4] = k1[e];
            vf[k][e] = v0[e];
            vf[k][e + 4] = v1[e];
          }
        } else {
          gu32x4 kk = gp<gu32x4>(a.k)[off / 8];
          gu32x4 vv = gp<gu32x4>(a.v)[off / 8];
          uint32_t kw[4] = {kk[0], kk[1], kk[2], kk[3]}, vw[4] = {vv[0], vv[1], vv[2], vv[3]};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            kf[k][2 * e] = __uint_as_float(kw[e] << 16);
            kf[k][2 * e + 1] = __uint_as_float(kw[e] & 0xffff0000u);
            vf[k][2 * e] = __uint_as_float(vw[e] << 16);
            vf[k][2 * e + 1] = __uint_as_float(vw[e] & 0xffff0000u);
          }
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) kf[k][e] = vf[k][e] = 0.0f;
      }
    }
#pragma unroll
    for (int u = 0; u < HG; ++u) {
      if (u >= Hg) break;
      float s[U];
#pragma unroll
      for (int k = 0; k < U; ++k) {
        float x = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) x += qv[u][e] * kf[k][e];
#pragma unroll
        for (int o = LPT / 2; o > 0; o >>= 1) x += __shfl_xor(x, o);
        s[k] = (tb + k < t1) ? x : -INFINITY;
      }
      float mt = s[0];
#pragma unroll
      for (int k = 1; k < U; ++k) mt = fmaxf(mt, s[k]);
      float mn = fmaxf(m[u], mt);
      float al = expf(m[u] - mn);
      float p[U], ps = 0.0f;
#pragma unroll
      for (int k = 0; k < U; ++k) {
        p[k] = expf(s[k] - mn);
        ps += p[k];
      }
      l[u] = al * l[u] + ps;
      m[u] = mn;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float x = al * acc[u][e];
#pragma unroll
        for (int k = 0; k < U; ++k) x += p[k] * vf[k][e];
        acc[u][e] = x;
      }
    }
  }
  // merge the lane groups of a wave (lanes 16 apart for D=128, 8 apart for D=64)
#pragma unroll
  for (int o = LPT; o < 64; o <<= 1) {
#pragma unroll
    for (int u = 0; u < HG; ++u) {
      float mo = __shfl_xor(m[u], o), lo = __shfl_xor(l[u], o);
      float mn = fmaxf(m[u], mo);
      float wa = (m[u] == -INFINITY) ? 0.0f : expf(m[u] - mn);
      float wb = (mo == -INFINITY) ? 0.0f : expf(mo - mn);
      l[u] = wa * l[u] + wb * lo;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[u][e] = wa * acc[u][e] + wb * __shfl_xor(acc[u][e], o);
      m[u] = mn;
    }
  }
  __shared__ float sm[4][HG], sl[4][HG], sacc[4][HG][D];
  const int wave = tid / 64, lane = tid % 64;
  if (lane < LPT) {
#pragma unroll
    for (int u = 0; u < HG; ++u) {
      if (lane == 0) {
        sm[wave][u] = m[u];
        sl[wave][u] = l[u];
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) sacc[wave][u][8 * lane + e] = acc[u][e];
    }
  }
  __syncthreads();
  for (int x = tid; x < Hg * D; x += 256) {
    int u = x / D, f = x % D;
    float mx = fmaxf(fmaxf(sm[0][u], sm[1][u]), fmaxf(sm[2][u], sm[3][u]));
    float ls = 0.0f, as = 0.0f;
    for (int w = 0; w < 4; ++w) {
      float wt = sm[w][u] == -INFINITY ? 0.0f : expf(sm[w][u] - mx);
      ls += wt * sl[w][u];
      as += wt * sacc[w][u][f];
    }
    float *part = a.ws + ((size_t)(b * a.H_q + h * Hg + u) * a.ws_splits + a.split0 + split) * (4 + D);
    if (f == 0) {
      part[0] = mx;
      part[1] = ls;
    }
    part[4 + f] = ls > 0.0f ? as / ls : 0.0f;
  }
}

// Flash-decoding over bf16 post-RoPE K and V with the scores on MFMA.
// Each wave takes 16 tokens per step: S^T (16 tokens x 16 query slots) =
// K Q^T on v_mfma_f32_16x16x32_bf16, K rows feeding the A operand straight
// from memory and the rotated query split into bf16 high and low parts (two
// products) so the scores carry ~16 mantissa bits of q.  The wave keeps its
// own online-softmax state; p goes through LDS to the lanes that own two
// output features each, which accumulate p V on VALU.  The next step's K and
// V are in flight while the current one is computed.
typedef __bf16 bf16x8d __attribute__((ext_vector_type(8)));
typedef float f32x4d __attribute__((ext_vector_type(4)));

template <int D, int HG>
__global__ __launch_bounds__(256, 2) void dense_mfma(DenseArgs a) {
  constexpr int KS = D / 32;          // K-steps of the score product
  constexpr int FPL = D / 64;         // output features per lane
  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  const int Hg = a.Hg, T = a.T;
  const int t0 = split * a.split_tokens, t1 = min(a.T_seq[b], t0 + a.split_tokens);
  __shared__ float qs[16][D];
  __shared__ float Pw[4][16][17];      // per wave: [token][query], padded
  __shared__ float Aw[4][16];          // per wave: rescale factor per query
  __shared__ float Mw[4][16], Lw[4][16];
  __shared__ float Ow[4][HG][D];

  for (int x = tid; x < 16 * (D / 2); x += 256) {
    const int u = x / (D / 2), i = x % (D / 2);
    float lo = 0.0f, hi = 0.0f;
    if (u < Hg) {
      const size_t qi = ((size_t)b * a.H_q + h * Hg + u) * D;
      float c, sn;
      rope_cs(a.q_pos[b], a.inv_freq[i], &c, &sn);
      const float xl = ldq(a.q, qi + i, a.q_f32), xh = ldq(a.q, qi + i + D / 2, a.q_f32);
      lo = (xl * c - xh * sn) * a.scale;
      hi = (xh * c + xl * sn) * a.scale;
    }
    qs[u][i] = lo;
    qs[u][i + D / 2] = hi;
  }
  __syncthreads();
  bf16x8d qh[KS], ql[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float x = qs[lr][32 * s + 8 * lg + j];
      const __bf16 hb = (__bf16)x;
      qh[s][j] = hb;
      ql[s][j] = (__bf16)(x - (float)hb);
    }

  gptr<bf16x8d> Kp = gp<bf16x8d>(a.k);
  gptr<uint32_t> Vp = gp<uint32_t>(a.v);
  const size_t base = ((size_t)b * a.H + h) * T;  // token rows of this head
  float m_w = -INFINITY, l_w = 0.0f;
  float acc[HG][FPL];
#pragma unroll
  for (int u = 0; u < HG; ++u)
#pragma unroll
    for (int e = 0; e < FPL; ++e) acc[u][e] = 0.0f;

  auto fetch = [&](int tb, bf16x8d (&kf)[KS], uint32_t (&vf)[16]) {
    const int tk = min(tb + lr, T - 1);
#pragma unroll
    for (int s = 0; s < KS; ++s) kf[s] = Kp[(base + tk) * (D / 8) + 4 * s + lg];
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const int tv = min(tb + t, T - 1);
      if constexpr (FPL == 2)
        vf[t] = Vp[(base + tv) * (D / 2) + lane];
      else
        vf[t] = (uint32_t)gp<uint16_t>(a.v)[(base + tv) * D + lane];
    }
  };
  bf16x8d kf[KS];
  uint32_t vf[16];
  int tb = t0 + 16 * wave;
  if (tb < t1) fetch(tb, kf, vf);
  for (int it = t0; it < t1; it += 64, tb += 64) {
    const bool live = tb < t1;
    bf16x8d kc[KS];
    uint32_t vc[16];
#pragma unroll
    for (int s = 0; s < KS; ++s) kc[s] = kf[s];
#pragma unroll
    for (int t = 0; t < 16; ++t) vc[t] = vf[t];
    if (tb + 64 < t1) fetch(tb + 64, kf, vf);
    float p[4] = {0, 0, 0, 0}, alpha = 1.0f;
    if (live) {
      f32x4d sacc = {0, 0, 0, 0};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kc[s], qh[s], sacc, 0, 0, 0);
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kc[s], ql[s], sacc, 0, 0, 0);
      }
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (tb + 4 * lg + i >= t1) sacc[i] = -INFINITY;
        mx = fmaxf(mx, sacc[i]);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mn = fmaxf(m_w, mx);
      alpha = __expf(m_w - mn);
      m_w = mn;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[i] = __expf(sacc[i] - mn);
        l_w = (i == 0 ? alpha * l_w : l_w) + p[i];
        Pw[wave][4 * lg + i][lr] = p[i];
      }
      if (lg == 0) Aw[wave][lr] = alpha;
    }
    __syncthreads();
    if (live) {
#pragma unroll
      for (int u = 0; u < HG; ++u) {
        const float al = Aw[wave][u];
#pragma unroll
        for (int e = 0; e < FPL; ++e) acc[u][e] *= al;
      }
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        float v0, v1 = 0.0f;
        if constexpr (FPL == 2) {
          v0 = __uint_as_float(vc[t] << 16);
          v1 = __uint_as_float(vc[t] & 0xffff0000u);
        } else {
          v0 = __uint_as_float(vc[t] << 16);
        }
#pragma unroll
        for (int u = 0; u < HG; ++u) {
          const float pu = Pw[wave][t][u];
          acc[u][0] += pu * v0;
          if constexpr (FPL == 2) acc[u][1] += pu * v1;
        }
      }
    }
    __syncthreads();
  }
  // combine the waves
  l_w += __shfl_xor(l_w, 16);
  l_w += __shfl_xor(l_w, 32);
  if (lg == 0) {
    Mw[wave][lr] = m_w;
    Lw[wave][lr] = l_w;
  }
#pragma unroll
  for (int u = 0; u < HG; ++u)
#pragma unroll
    for (int e = 0; e < FPL; ++e) Ow[wave][u][FPL * lane + e] = acc[u][e];
  __syncthreads();
  for (int x = tid; x < Hg * D; x += 256) {
    const int u = x / D, f = x % D;
    float mx = fmaxf(fmaxf(Mw[0][u], Mw[1][u]), fmaxf(Mw[2][u], Mw[3][u]));
    float ls = 0.0f, os = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float wt = Mw[w][u] == -INFINITY ? 0.0f : __expf(Mw[w][u] - mx);
      ls += wt * Lw[w][u];
      os += wt * Ow[w][u][f];
    }
    float *part = a.ws + ((size_t)(b * a.H_q + h * Hg + u) * a.ws_splits + a.split0 + split) * (4 + D);
    if (f == 0) {
      part[0] = mx;
      part[1] = ls;
    }
    part[4 + f] = ls > 0.0f ? os / ls : 0.0f;
  }
}

// Combine split partials [m, l, 0, 0, o[d]] (o divided by its split's l) of
// one (sequence, query head): o = sum_s w_s l_s o_s / sum_s w_s l_s with
// w_s = exp(m_s - max m).  The first 32 splits' columns are fetched together
// with m and l, so short reductions take one memory round trip.
__global__ __launch_bounds__(256) void merge_outputs(const float *ws, float *out, int ns, int d,
                                                     int H_q, float *stats) {
  const int j = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int st = 4 + d, f = tid & 127, part = tid >> 7;
  const float *pb = ws + ((size_t)(b * H_q + j) * ns) * st;
  __shared__ float m_s[kMaxSplits], w_s[kMaxSplits];
  __shared__ float red[8];
  __shared__ float half_s[kMaxD];
  float v[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int s = part + 2 * k;
    v[k] = (f < d && s < ns) ? pb[(size_t)s * st + 4 + f] : 0.0f;
  }
  float mx = -INFINITY;
  for (int s = tid; s < ns; s += 256) {
    const float m = pb[(size_t)s * st], l = pb[(size_t)s * st + 1];
    m_s[s] = m;
    w_s[s] = l;
    mx = fmaxf(mx, m);
  }
  mx = block_reduce(mx, red, true);
  float ls = 0.0f;
  for (int s = tid; s < ns; s += 256) {
    const float m = m_s[s];
    const float w = m == -INFINITY ? 0.0f : __expf(m - mx) * w_s[s];
    w_s[s] = w;
    ls += w;
  }
  ls = block_reduce(ls, red, false);
  float acc = 0.0f;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int s = part + 2 * k;
    if (s < ns && w_s[s] > 0.0f) acc += w_s[s] * v[k];  // empty splits carry no payload
  }
  for (int s0 = 32; s0 < ns; s0 += 32) {
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int s = s0 + part + 2 * k;
      v[k] = (f < d && s < ns) ? pb[(size_t)s * st + 4 + f] : 0.0f;
    }
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int s = s0 + part + 2 * k;
      if (s < ns && w_s[s] > 0.0f) acc += w_s[s] * v[k];
    }
  }
  if (part == 1 && f < d) half_s[f] = acc;
  __syncthreads();
  if (part == 0 && f < d) out[((size_t)b * H_q + j) * d + f] = (acc + half_s[f]) / ls;
  if (stats && tid == 0) {
    stats[((size_t)b * H_q + j) * 2] = mx;
    stats[((size_t)b * H_q + j) * 2 + 1] = ls;
  }
}

// ------------------------------------------------------------- unpack --
__global__ void unpack_codes(const LayerDev *layer, int tau, int H, int T, int d, uint8_t *out) {
  const LayerDev &L = *layer;
  const CellDev &c = L.c[tau];
  size_t n = (size_t)H * T * d;
  for (size_t x = blockIdx.x * (size_t)blockDim.x + threadIdx.x; x < n;
       x += (size_t)gridDim.x * blockDim.x) {
    int i = x % d;
    int t = (x / d) % T;
    int h = x / ((size_t)d * T);
    out[x] = (uint8_t)(tau == 0 ? k_code(c, h, t, i, L.T_pad, d) : v_code(c, h, t, i, L.T_pad, d));
  }
}

__global__ void sincos_kernel(const float *x, int n, float *sn, float *cs, int variant) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) {
    if (variant == 1)
      hw_sincos(x[i], sn + i, cs + i);
    else if (variant == 2)  // (position, inv_freq) pairs, as the key path's small-angle blocks
      rope_rev_cs_hw(x[2 * i], x[2 * i + 1] * kInv2Pi, cs + i, sn + i);
    else
      fast_sincos(x[i], sn + i, cs + i);
  }
}

}  // namespace

hipError_t jolt_launch_sincos(const float *x, int n, float *sn, float *cs, int variant,
                              hipStream_t s) {
  hipLaunchKernelGGL(sincos_kernel, dim3((n + 255) / 256), dim3(256), 0, s, x, n, sn, cs, variant);
  return hipGetLastError();
}

hipError_t jolt_launch_generic(const DecodeArgs &a, int nseq, hipStream_t s, KernelEvents ev) {
  dim3 grid(a.n_split, a.H, nseq);
  auto k = a.f32 ? decode_generic<true> : decode_generic<false>;
  if (ev.begin || ev.end)  // events take the kernel's own start / end timestamps
    hipExtLaunchKernelGGL(k, grid, dim3(256), 0u, s, ev.begin, ev.end, 0u, a);
  else
    hipLaunchKernelGGL(k, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t jolt_launch_merge(const DecodeArgs &a, int nseq, hipStream_t s) {
  dim3 grid(a.H_q, nseq);
  if (a.f32)
    hipLaunchKernelGGL(merge_finalize<true>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(merge_finalize<false>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int D, bool KV32>
static void launch_dense_hg(const DenseArgs &a, dim3 grid, hipStream_t s) {
  if (a.Hg <= 1)
    hipLaunchKernelGGL((dense_split<D, 1, KV32>), grid, dim3(256), 0, s, a);
  else if (a.Hg <= 2)
    hipLaunchKernelGGL((dense_split<D, 2, KV32>), grid, dim3(256), 0, s, a);
  else if (a.Hg <= 4)
    hipLaunchKernelGGL((dense_split<D, 4, KV32>), grid, dim3(256), 0, s, a);
  else if (a.Hg <= 8)
    hipLaunchKernelGGL((dense_split<D, 8, KV32>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((dense_split<D, 16, KV32>), grid, dim3(256), 0, s, a);
}

template <int D>
static void launch_dense_mfma(const DenseArgs &a, dim3 grid, hipStream_t s) {
  if (a.Hg <= 4)
    hipLaunchKernelGGL((dense_mfma<D, 4>), grid, dim3(256), 0, s, a);
  else if (a.Hg <= 8)
    hipLaunchKernelGGL((dense_mfma<D, 8>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((dense_mfma<D, 16>), grid, dim3(256), 0, s, a);
}

hipError_t jolt_launch_dense(const DenseArgs &a, int nseq, hipStream_t s) {
  dim3 grid(a.n_split, a.H, nseq);
  if (!a.kv_f32) {
    if (a.d == 128)
      launch_dense_mfma<128>(a, grid, s);
    else
      launch_dense_mfma<64>(a, grid, s);
    return hipGetLastError();
  }
  if (a.d == 128)
    a.kv_f32 ? launch_dense_hg<128, true>(a, grid, s) : launch_dense_hg<128, false>(a, grid, s);
  else
    a.kv_f32 ? launch_dense_hg<64, true>(a, grid, s) : launch_dense_hg<64, false>(a, grid, s);
  return hipGetLastError();
}

hipError_t jolt_launch_dense_merge(const DenseArgs &a, int nseq, hipStream_t s) {
  hipLaunchKernelGGL(merge_outputs, dim3(a.H_q, nseq), dim3(256), 0, s, (const float *)a.ws, a.out,
                     a.ws_splits, a.d, a.H_q, (float *)nullptr);
  return hipGetLastError();
}

// ns: splits per (sequence, query head) row of the workspace (the split
// kernel's plus any uncompressed-tail splits)
hipError_t jolt_launch_merge_outputs(const DecodeArgs &a, int nseq, int ns, hipStream_t s,
                                     float *stats) {
  hipLaunchKernelGGL(merge_outputs, dim3(a.H_q, nseq), dim3(256), 0, s, (const float *)a.ws, a.out,
                     ns, a.d, a.H_q, stats);
  return hipGetLastError();
}

hipError_t jolt_launch_unpack(const LayerDev *layer, int tau, int H, int T, int d, uint8_t *out,
                              hipStream_t s) {
  size_t n = (size_t)H * T * d;
  int blocks = (int)((n + 255) / 256);
  if (blocks > 65535) blocks = 65535;
  hipLaunchKernelGGL(unpack_codes, dim3(blocks), dim3(256), 0, s, layer, tau, H, T, d, out);
  return hipGetLastError();
}
