// Dispatch of the MFMA decode kernel (decode_mfma.inc) by key/value bits.
#include <hip/hip_runtime.h>

#include "jolt_internal.h"

namespace jolt_mfma {
hipError_t launch_bk0(const jolt::DecodeArgs &, int, int, int, int, int, hipStream_t);
hipError_t launch_bk2(const jolt::DecodeArgs &, int, int, int, int, int, hipStream_t);
hipError_t launch_bk4(const jolt::DecodeArgs &, int, int, int, int, int, hipStream_t);
hipError_t launch_bk8(const jolt::DecodeArgs &, int, int, int, int, int, hipStream_t);
}  // namespace jolt_mfma

// nkt: key-rank steps of 32, nmv: value-rank blocks of 16 (maxima over the
// sequences of the launch).
hipError_t jolt_launch_mfma(const jolt::DecodeArgs &a, int nseq, int bK, int bV, int nkt,
                            int lds_bytes, hipStream_t s) {
  const int nvb = a.rV_max / 16;
  switch (bK) {
    case 0: return jolt_mfma::launch_bk0(a, nseq, bV, nkt, nvb, lds_bytes, s);
    case 2: return jolt_mfma::launch_bk2(a, nseq, bV, nkt, nvb, lds_bytes, s);
    case 4: return jolt_mfma::launch_bk4(a, nseq, bV, nkt, nvb, lds_bytes, s);
    default: return jolt_mfma::launch_bk8(a, nseq, bV, nkt, nvb, lds_bytes, s);
  }
}

// LDS available to one workgroup on gfx950 (160 KiB per CU).
int jolt_mfma_max_lds() { return 160 * 1024; }
