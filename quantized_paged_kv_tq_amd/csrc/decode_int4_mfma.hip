// INT4 split-KV decode, stage 1, on the matrix cores (placeholder until the
// MFMA kernel lands: reports "not supported" so the generic kernel runs).
#include "tq_internal.h"

namespace tqk {
hipError_t launch_decode_int4_mfma(const DecodeParams&, hipStream_t) {
  return hipErrorNotSupported;
}
}  // namespace tqk
