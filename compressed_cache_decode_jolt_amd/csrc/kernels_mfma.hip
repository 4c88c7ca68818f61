// MFMA split-T decode kernel (gfx950) -- not built yet.
#include <hip/hip_runtime.h>

#include "jolt_internal.h"

hipError_t jolt_launch_mfma(const jolt::DecodeArgs &, int, int, int, int, hipStream_t) {
  return hipErrorInvalidValue;
}
int jolt_mfma_max_lds() { return 0; }
