// Instantiations of the MFMA decode kernel for 8-bit key and 2-bit value residuals.
#include "mfma_launch.inc"

namespace jolt_mfma {
hipError_t launch_k8_v2(const jolt::MfmaArgs &a, int nseq, int nkt, int nmv, int lds,
                          hipStream_t s, jolt::KernelEvents ev) {
  return launch_bits<8, 2>(a, nseq, nkt, nmv, lds, s, ev);
}
}  // namespace jolt_mfma
