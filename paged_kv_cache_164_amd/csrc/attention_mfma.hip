// Paged decode attention, phase 1, matrix-core variant for grouped-query heads (placeholder).
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

bool mfma_supported(int, int, int, int) { return false; }

hipError_t launch_decode_mfma(const DecodeArgs&, int, int, int, int, hipStream_t) {
  return hipErrorInvalidValue;
}

}  // namespace pkv
