// Dispatch of the MFMA decode kernel (decode_mfma.inc) by key/value bits.
#include <hip/hip_runtime.h>

#include "jolt_internal.h"

namespace jolt_mfma {
hipError_t launch_k0_v0(const jolt::MfmaArgs &, int, int, int, int, hipStream_t, jolt::KernelEvents);
hipError_t launch_k0_v2(const jolt::MfmaArgs &, int, int, int, int, hipStream_t, jolt::KernelEvents);
hipError_t launch_k0_v4(const jolt::MfmaArgs &, int, int, int, int, hipStream_t, jolt::KernelEvents);
hipError_t launch_k0_v8(const jolt::MfmaArgs &, int, int, int, int, hipStream_t, jolt::KernelEvents);
hipError_t launch_k2_v0(const jolt::MfmaArgs &, int, int, int, int, hipStream_t, jolt::KernelEvents);
hipError_t launch_k2_v2(const jolt::MfmaArgs &, int, int, int, int, hipStream_t, jolt::KernelEvents);
hipError_t launch_k2_v4(const jolt::MfmaArgs &, int, int, int, int, hipStream_t, jolt::KernelEvents);
hipError_t launch_k2_v8(const jolt::MfmaArgs &, int, int, int, int, hipStream_t, jolt::KernelEvents);
hipError_t launch_k4_v0(const jolt::MfmaArgs &, int, int, int, int, hipStream_t, jolt::KernelEvents);
hipError_t launch_k4_v2(const jolt::MfmaArgs &, int, int, int, int, hipStream_t, jolt::KernelEvents);
hipError_t launch_k4_v4(const jolt::MfmaArgs &, int, int, int, int, hipStream_t, jolt::KernelEvents);
hipError_t launch_k4_v8(const jolt::MfmaArgs &, int, int, int, int, hipStream_t, jolt::KernelEvents);
hipError_t launch_k8_v0(const jolt::MfmaArgs &, int, int, int, int, hipStream_t, jolt::KernelEvents);
hipError_t launch_k8_v2(const jolt::MfmaArgs &, int, int, int, int, hipStream_t, jolt::KernelEvents);
hipError_t launch_k8_v4(const jolt::MfmaArgs &, int, int, int, int, hipStream_t, jolt::KernelEvents);
hipError_t launch_k8_v8(const jolt::MfmaArgs &, int, int, int, int, hipStream_t, jolt::KernelEvents);
}  // namespace jolt_mfma

// nkt: key-rank steps of 32 (the same for every sequence of the launch);
// the value-rank blocks of 16 are the launch's maximum.
hipError_t jolt_launch_mfma(const jolt::MfmaArgs &a, int nseq, int bK, int bV, int nkt,
                            int lds_bytes, hipStream_t s, jolt::KernelEvents ev) {
  using namespace jolt_mfma;
  typedef hipError_t (*fn)(const jolt::MfmaArgs &, int, int, int, int, hipStream_t,
                           jolt::KernelEvents);
  static const fn table[4][4] = {
      {launch_k0_v0, launch_k0_v2, launch_k0_v4, launch_k0_v8},
      {launch_k2_v0, launch_k2_v2, launch_k2_v4, launch_k2_v8},
      {launch_k4_v0, launch_k4_v2, launch_k4_v4, launch_k4_v8},
      {launch_k8_v0, launch_k8_v2, launch_k8_v4, launch_k8_v8}};
  auto idx = [](int b) { return b == 0 ? 0 : b == 2 ? 1 : b == 4 ? 2 : 3; };
  return table[idx(bK)][idx(bV)](a, nseq, nkt, a.rV_max / 16, lds_bytes, s, ev);
}

// LDS available to one workgroup on gfx950 (160 KiB per CU).
int jolt_mfma_max_lds() { return 160 * 1024; }
