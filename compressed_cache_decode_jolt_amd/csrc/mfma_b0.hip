// Instantiations of the MFMA decode kernel for 0-bit key residuals.
#include "decode_mfma.inc"

namespace jolt_mfma {

template <int BV, int KT, int NVB>
static hipError_t go(const jolt::DecodeArgs &a, int nseq, int lds, hipStream_t s) {
  auto k = decode_mfma<0, BV, KT, NVB>;
  static bool attr = false;
  if (!attr) {
    hipError_t e = hipFuncSetAttribute((const void *)k, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       160 * 1024);
    if (e != hipSuccess) return e;
    attr = true;
  }
  dim3 grid((unsigned)(nseq * a.n_split * a.H));
  hipLaunchKernelGGL(k, grid, dim3(256), lds, s, a);
  return hipGetLastError();
}

// size classes (key r_T steps, value-rank blocks per wave): (2,2), (8,2), (8,8)
template <int BV>
static hipError_t go_v(const jolt::DecodeArgs &a, int nseq, int nkt, int nvb, int lds,
                       hipStream_t s) {
  if (nvb > 2) return go<BV, 8, 8>(a, nseq, lds, s);
  if (nkt > 2) return go<BV, 8, 2>(a, nseq, lds, s);
  return go<BV, 2, 2>(a, nseq, lds, s);
}

hipError_t launch_bk0(const jolt::DecodeArgs &a, int nseq, int bV, int nkt, int nvb, int lds,
                       hipStream_t s) {
  switch (bV) {
    case 0: return go_v<0>(a, nseq, nkt, nvb, lds, s);
    case 2: return go_v<2>(a, nseq, nkt, nvb, lds, s);
    case 4: return go_v<4>(a, nseq, nkt, nvb, lds, s);
    default: return go_v<8>(a, nseq, nkt, nvb, lds, s);
  }
}

}  // namespace jolt_mfma
