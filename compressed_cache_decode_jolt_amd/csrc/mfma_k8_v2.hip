// Instantiations of the MFMA decode kernel for 8-bit key and 2-bit value residuals.
#include "decode_mfma.inc"

namespace jolt_mfma {

template <int KT, int MV, int WAVES, int NB>
static hipError_t go(const jolt::MfmaArgs &a, int nseq, int lds, hipStream_t s) {
  auto k = decode_mfma<8, 2, KT, MV, WAVES, NB>;
  static bool attr = false;
  if (!attr) {
    hipError_t e = hipFuncSetAttribute((const void *)k, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       160 * 1024);
    if (e != hipSuccess) return e;
    attr = true;
  }
  const dim3 grid = a.grid8 ? dim3((unsigned)(8 * a.H), (unsigned)(a.n_split / 8), (unsigned)nseq)
                            : dim3((unsigned)a.H, (unsigned)a.n_split, (unsigned)nseq);
  hipLaunchKernelGGL(k, grid, dim3(64 * WAVES), lds, s, a);
  return hipGetLastError();
}

// value classes: ranks <= 64 or <= 128 with 8 waves (two per SIMD), <= 512
// with 4 waves holding the accumulators of 32 rank blocks each.  Key ranks
// above 256 (more than 8 steps; padded to 64, so the step count is even)
// always run 4 waves: their W2_K fills the LDS and Pi's fragments move to
// registers; with them, value ranks up to 256.
template <int KT>
static hipError_t go_kt(const jolt::MfmaArgs &a, int nseq, int nmv, int lds, hipStream_t s) {
  if constexpr (KT > 8) {  // value ranks <= 256 (the host sends wider ones elsewhere)
    if (nmv > 8) return go<KT, 16, 4, 1>(a, nseq, lds, s);
    if (nmv > 4) return go<KT, 8, 4, 1>(a, nseq, lds, s);
    return go<KT, 4, 4, 1>(a, nseq, lds, s);
  } else {
    if (nmv > 8) return go<KT, 32, 4, 1>(a, nseq, lds, s);
    if (nmv > 4) return go<KT, 8, 8, 1>(a, nseq, lds, s);
    return go<KT, 4, 8, 1>(a, nseq, lds, s);
  }
}

// nkt: exact key-rank steps of 32 (0..8, 10, 12, 14, 16)
hipError_t launch_k8_v2(const jolt::MfmaArgs &a, int nseq, int nkt, int nmv, int lds,
                          hipStream_t s) {
  switch (nkt) {
    case 0: return go_kt<0>(a, nseq, nmv, lds, s);
    case 1: return go_kt<1>(a, nseq, nmv, lds, s);
    case 2: return go_kt<2>(a, nseq, nmv, lds, s);
    case 3: return go_kt<3>(a, nseq, nmv, lds, s);
    case 4: return go_kt<4>(a, nseq, nmv, lds, s);
    case 5: return go_kt<5>(a, nseq, nmv, lds, s);
    case 6: return go_kt<6>(a, nseq, nmv, lds, s);
    case 7: return go_kt<7>(a, nseq, nmv, lds, s);
    case 8: return go_kt<8>(a, nseq, nmv, lds, s);
    case 10: return go_kt<10>(a, nseq, nmv, lds, s);
    case 12: return go_kt<12>(a, nseq, nmv, lds, s);
    case 14: return go_kt<14>(a, nseq, nmv, lds, s);
    case 16: return go_kt<16>(a, nseq, nmv, lds, s);
    default: return hipErrorInvalidValue;  // odd step counts above 8 are never planned
  }
}

}  // namespace jolt_mfma
