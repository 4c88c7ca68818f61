// Instantiations of the MFMA decode kernel for 0-bit key residuals.
#include "decode_mfma.inc"

namespace jolt_mfma {

template <int BV, int KT, int MV, int WAVES>
static hipError_t go(const jolt::DecodeArgs &a, int nseq, int lds, hipStream_t s) {
  auto k = decode_mfma<0, BV, KT, MV, WAVES>;
  static bool attr = false;
  if (!attr) {
    hipError_t e = hipFuncSetAttribute((const void *)k, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       160 * 1024);
    if (e != hipSuccess) return e;
    attr = true;
  }
  dim3 grid((unsigned)(nseq * a.n_split * a.H));
  hipLaunchKernelGGL(k, grid, dim3(64 * WAVES), lds, s, a);
  return hipGetLastError();
}

// size classes: key r_T steps of 32 held in registers (2, 4, 8) x value
// ranks (<= 64 or <= 128: 8 waves, two per SIMD; <= 512: 4 waves with the
// accumulators of 32 rank blocks each)
template <int BV>
static hipError_t go_v(const jolt::DecodeArgs &a, int nseq, int nkt, int nmv, int lds,
                       hipStream_t s) {
  if (nmv > 8) {
    if (nkt > 4) return go<BV, 8, 32, 4>(a, nseq, lds, s);
    if (nkt > 2) return go<BV, 4, 32, 4>(a, nseq, lds, s);
    return go<BV, 2, 32, 4>(a, nseq, lds, s);
  }
  if (nmv > 4) {
    if (nkt > 4) return go<BV, 8, 8, 8>(a, nseq, lds, s);
    if (nkt > 2) return go<BV, 4, 8, 8>(a, nseq, lds, s);
    return go<BV, 2, 8, 8>(a, nseq, lds, s);
  }
  if (nkt > 4) return go<BV, 8, 4, 8>(a, nseq, lds, s);
  if (nkt > 2) return go<BV, 4, 4, 8>(a, nseq, lds, s);
  return go<BV, 2, 4, 8>(a, nseq, lds, s);
}

hipError_t launch_bk0(const jolt::DecodeArgs &a, int nseq, int bV, int nkt, int nmv, int lds,
                       hipStream_t s) {
  switch (bV) {
    case 0: return go_v<0>(a, nseq, nkt, nmv, lds, s);
    case 2: return go_v<2>(a, nseq, nkt, nmv, lds, s);
    case 4: return go_v<4>(a, nseq, nkt, nmv, lds, s);
    default: return go_v<8>(a, nseq, nkt, nmv, lds, s);
  }
}

}  // namespace jolt_mfma
