// Branch-free float32 sine and cosine for RoPE angles (device code).
//
// RoPE rotates each key and query pair by the float32 angle fl32(t * inv_freq)
// built in-kernel from int32 positions (the sarnas.ru JoLT post, section on
// building cos/sin inside the kernel: float32 is required because angles reach
// ~1e5 rad at 128K tokens).  The decode path needs one sine/cosine pair per
// (token, feature pair, KV head), so it uses this short evaluation instead of
// the general library routine:
//
//   1. Cody-Waite reduction (W. J. Cody and W. Waite, "Software Manual for the
//      Elementary Functions", 1980): k = rint(x * 2/pi) and
//      r = x - k pi/2 with pi/2 split into three float32 parts
//      C1 + C2 + C3 (C1 = fl32(pi/2), C2 = fl32(pi/2 - C1),
//      C3 = fl32(pi/2 - C1 - C2)), each step one fused multiply-add.  For
//      |x| < 2^20 the first step is exact (x - k C1 is a multiple of 2^-23
//      below 1) and |r| <= pi/4 + 0.04.
//   2. Taylor polynomials of sin and cos on that interval, through x^11 and
//      x^10 (truncation error < 3e-10), evaluated by Horner's rule.
//   3. Quadrant k mod 4 selects and negates.
// Accuracy is pinned by a GPU test against float64 over all angles of
// positions 0..65536 and over random angles up to 2^20.
#pragma once
#include <hip/hip_runtime.h>

namespace jolt {

// 1 / (2 pi) rounded to float32: radians -> revolutions for the hardware units
constexpr float kInv2Pi = 0.15915493667125702f;


// Domain: |x| < 2^20.  The host enforces it (positions <= 2^20 and
// 0 <= inv_freq <= 1, true of every RoPE frequency schedule).
__device__ inline void fast_sincos(float x, float *s, float *c) {
  const float kf = __builtin_rintf(x * 0.636619746685028076171875f);
  float r = __builtin_fmaf(-kf, 1.57079637050628662109375f, x);
  r = __builtin_fmaf(-kf, -4.37113882867379300296306610107421875e-08f, r);
  r = __builtin_fmaf(-kf, -1.71512451000588189e-15f, r);
  const float r2 = r * r;
  float sp = -2.5052107943679403e-08f;
  sp = __builtin_fmaf(sp, r2, 2.7557318844628753e-06f);
  sp = __builtin_fmaf(sp, r2, -1.9841270113829523e-04f);
  sp = __builtin_fmaf(sp, r2, 8.3333337679505348e-03f);
  sp = __builtin_fmaf(sp, r2, -1.6666667163372040e-01f);
  const float sr = __builtin_fmaf(sp * r2, r, r);
  float cp = -2.755731998149713e-07f;
  cp = __builtin_fmaf(cp, r2, 2.4801587642286904e-05f);
  cp = __builtin_fmaf(cp, r2, -1.3888889225199819e-03f);
  cp = __builtin_fmaf(cp, r2, 4.1666667908430099e-02f);
  cp = __builtin_fmaf(cp, r2, -0.5f);
  const float cr = __builtin_fmaf(cp, r2, 1.0f);
  const int q = (int)kf;
  const float s0 = (q & 1) ? cr : sr;
  const float c0 = (q & 1) ? sr : cr;
  *s = __uint_as_float(__float_as_uint(s0) ^ ((uint32_t)(q & 2) << 30));
  *c = __uint_as_float(__float_as_uint(c0) ^ ((uint32_t)((q + 1) & 2) << 30));
}

// cos/sin of the RoPE angle of feature pair i at position t.
__device__ inline void rope_angle_cs(int t, float inv_freq, float *c, float *s) {
  fast_sincos(__fmul_rn((float)t, inv_freq), s, c);
}

// Shorter variant for the bf16/fp16 MFMA path (max error ~5e-7, well inside
// what fp16 operands carry): Cody-Waite reduction by 2 pi in two float32
// parts (C1 = fl32(2 pi) = 13176795 * 2^-21, so x - k C1 is exact for
// |x| < 2^20: both terms are multiples of 2^-21, or k = 0; the remainder of
// 2 pi - C1 - C2 is 6.9e-15, so the term dropped is below 1.2e-9 over the
// domain), then the hardware sine and cosine units, which take the angle in
// revolutions.  Same domain as fast_sincos.
__device__ inline void hw_sincos(float x, float *s, float *c) {
  const float k = __builtin_rintf(x * kInv2Pi);
  float r = __builtin_fmaf(-k, 6.2831854820251465f, x);
  r = __builtin_fmaf(-k, -1.7484555314695172e-07f, r);
  const float rev = r * kInv2Pi;
  *s = __builtin_amdgcn_sinf(rev);
  *c = __builtin_amdgcn_cosf(rev);
}

__device__ inline void rope_angle_cs_hw(int t, float inv_freq, float *c, float *s) {
  hw_sincos(__fmul_rn((float)t, inv_freq), s, c);
}

// Angles known to stay below 128 rad (about 20 revolutions): the position
// times inv_freq / (2 pi) goes to the hardware units directly.  Against
// sin/cos of fl32(t * inv_freq) this adds at most three float32 roundings of
// a value below 20.4, i.e. under 2.3e-5 rad -- a tenth of what the fp16 key
// operands carry.
__device__ inline void rope_rev_cs_hw(float t, float inv_freq_rev, float *c, float *s) {
  const float rev = t * inv_freq_rev;
  *s = __builtin_amdgcn_sinf(rev);
  *c = __builtin_amdgcn_cosf(rev);
}

}  // namespace jolt
