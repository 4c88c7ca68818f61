// Instantiations of the MFMA decode kernel for 0-bit key and 8-bit value residuals.
#include "mfma_launch.inc"

namespace jolt_mfma {
hipError_t launch_k0_v8(const jolt::MfmaArgs &a, int nseq, int nkt, int nmv, int lds,
                          hipStream_t s, jolt::KernelEvents ev) {
  return launch_bits<0, 8>(a, nseq, nkt, nmv, lds, s, ev);
}
}  // namespace jolt_mfma
