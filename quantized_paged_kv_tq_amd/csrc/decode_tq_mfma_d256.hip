// TurboQuant split-KV decode, stage 1, on the CDNA4 matrix cores: the
// FP8-key kernel's launches at head dim 256 (decode_tq_kernel.h); the
// caller has set the workgroup layout (four query heads per wave).
#include "decode_tq_kernel.h"

namespace tqk {

hipError_t launch_decode_tq_d256(DecodeParams& p, hipStream_t st, bool wide) {
  switch (p.wgh * ((p.g + 3) / 4)) {
    case 1: return launch<1, 1, 256>(p, st, wide);
    case 2: return launch<2, 1, 256>(p, st, wide);
    default: return launch<4, 1, 256>(p, st, wide);
  }
}

}  // namespace tqk
